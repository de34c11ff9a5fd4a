"""Parity of attention_bf16 (softmax(scale Q K^T) V per head, the chain of two
products the "Tensor Cores" chapter (ai-infra-handbooks), section "mma.sync:
the register layout is explicit", names as FlashAttention's) against the
oracle.

Tolerance, from the arithmetic of the kernel.  The weights are rounded to
BF16 for the second product while the row sum uses the FP32 weights.  BF16
keeps 8 significant bits (1/8/7 split, "Tensor Cores" chapter, section
"Precision"), so round-to-nearest moves a weight by up to 2^-8 of itself
(0.502 becomes 0.50390625), and O by at most 2^-8 sum_j w_j |v_j| / l =
2^-8 A (A from the oracle).  The
FP32 scores carry at most scale (d + 4) 2^-23 max_j sum_k |q_k k_jk| of
error into the exponent, which moves every weight ratio by twice that.  The
output is rounded to BF16 once (2^-8 |O| with slack), and 2^-16 A covers the
hardware exp2 and reciprocal.  lse: the exponent error plus Sk 2^-23 for the
FP32 row sum."""
import numpy as np
import pytest
import torch

import dense_matrix_unit_amd as dmu
import oracle
from dense_matrix_unit_amd import workloads as wl

pytestmark = pytest.mark.gpu


def bf16(shape, seed, mult=1.0):
    return oracle.encode_bf16((wl.normal(shape, seed) * np.float32(mult)).astype(np.float32))


def to_gpu(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def from_gpu(t):
    return oracle.decode_bf16(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def expo_err(Q, K, scale, d):
    q = np.abs(oracle.decode_bf16(Q))
    k = np.abs(oracle.decode_bf16(K))
    return scale * (d + 4) * 2.0 ** -23 * (q @ np.swapaxes(k, -1, -2)).max(axis=-1)


def check(O, lse, Q, K, V, scale, causal, what):
    d = Q.shape[-1]
    Oref, lref, A = oracle.attention_bf16(Q, K, V, scale, causal)
    e = expo_err(Q, K, scale, d)[..., None]
    tol = A * (2.0 ** -8 + 2.0 ** -16 + 2 * e) + 2.0 ** -8 * np.abs(Oref) + 1e-30
    bad = ~(np.abs(O - Oref) <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d outside; first %s got %r want %r tol %r"
                             % (what, bad.sum(), bad.size, i, O[i], Oref[i], tol[i]))
    if lse is not None:
        Sk = K.shape[-2]
        tl = e[..., 0] + Sk * 2.0 ** -23 + 2.0 ** -20 * np.abs(lref)
        assert np.all(np.abs(lse - lref) <= tl), "%s: lse" % what


def run(Q, K, V, scale, causal, with_lse=True):
    heads, Sq, d = Q.shape
    O = torch.empty((heads, Sq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((heads, Sq), dtype=torch.float32, device="cuda") if with_lse else None
    dmu.attention_bf16(to_gpu(Q), to_gpu(K), to_gpu(V), O, scale, causal, lse)
    torch.cuda.synchronize()
    return from_gpu(O), (lse.cpu().numpy().astype(np.float64) if with_lse else None)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 128, 128, 128), (2, 200, 300, 128), (3, 65, 130, 64),
                                   (2, 256, 256, 64), (1, 1, 1, 128), (1, 3, 700, 128),
                                   (2, 129, 129, 128), (2, 640, 700, 128)])
def test_attention_matches_oracle(shape, causal):
    # ragged query blocks (Sq % 128) and key blocks (Sk % 64), one-row and
    # one-key heads, Sq < Sk under the causal mask; with the mask a workgroup
    # takes a pair of query blocks, and an odd count leaves a middle block
    # alone (Sq = 300, 640)
    heads, Sq, Sk, d = shape
    Q, K, V = bf16((heads, Sq, d), 1), bf16((heads, Sk, d), 2), bf16((heads, Sk, d), 3)
    scale = 1.0 / np.sqrt(d)
    O, lse = run(Q, K, V, scale, causal)
    check(O, lse, Q, K, V, scale, causal, "%s causal %s" % (shape, causal))


def test_attention_large_scores():
    # scores in the hundreds: the running maximum moves often and far
    Q, K, V = bf16((2, 256, 128), 4, 4.0), bf16((2, 512, 128), 5, 4.0), bf16((2, 512, 128), 6)
    O, lse = run(Q, K, V, 0.125, False)
    check(O, lse, Q, K, V, 0.125, False, "large scores")


def test_attention_single_visible_key_is_exact():
    # one key: weight exp2(0) = 1, sum 1, O = V[0] exactly
    Q, K, V = bf16((2, 100, 64), 7), bf16((2, 1, 64), 8), bf16((2, 1, 64), 9)
    O, _ = run(Q, K, V, 0.3, False, with_lse=False)
    assert np.array_equal(O, np.broadcast_to(oracle.decode_bf16(V), O.shape))
    # causal, Sq == Sk: row 0 sees key 0 only
    Q, K, V = bf16((2, 150, 128), 10), bf16((2, 150, 128), 11), bf16((2, 150, 128), 12)
    O, _ = run(Q, K, V, 0.1, True, with_lse=False)
    assert np.array_equal(O[:, 0], oracle.decode_bf16(V[:, 0]))


def test_attention_strided_heads():
    # [S, heads, d] storage: head stride d, row stride heads * d, for all four
    H, Sq, Sk, d = 4, 190, 250, 128
    Qf, Kf, Vf = bf16((Sq, H, d), 13), bf16((Sk, H, d), 14), bf16((Sk, H, d), 15)
    Qg, Kg, Vg = (to_gpu(x).permute(1, 0, 2) for x in (Qf, Kf, Vf))
    Og = torch.empty((Sq, H, d), dtype=torch.bfloat16, device="cuda").permute(1, 0, 2)
    lse = torch.empty((H, Sq), dtype=torch.float32, device="cuda")
    dmu.attention_bf16(Qg, Kg, Vg, Og, 0.09, True, lse)
    torch.cuda.synchronize()
    O = from_gpu(Og)
    Q, K, V = (np.ascontiguousarray(x.transpose(1, 0, 2)) for x in (Qf, Kf, Vf))
    check(O, lse.cpu().numpy().astype(np.float64), Q, K, V, 0.09, True, "strided")


@pytest.mark.parametrize("causal", [False, True])
def test_attention_workload(causal):
    # the benchmark's shape (32 heads of 4096 x 4096, d = 128) in full: every
    # output row of every head against the oracle, one head at a time
    H, S, d = 32, 4096, 128
    Q = bf16((H, S, d), 21)
    K = bf16((H, S, d), 22)
    V = bf16((H, S, d), 23)
    scale = 1.0 / np.sqrt(d)
    O, lse = run(Q, K, V, scale, causal)
    for h in range(H):
        sl = np.s_[h:h + 1]
        check(O[sl], lse[sl], Q[sl], K[sl], V[sl], scale, causal, "head %d" % h)


def test_attention_rejects_bad_arguments():
    Q = torch.zeros((1, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dmu.DmuError):
        dmu.attention_bf16(Q, Q, Q, torch.empty_like(Q), 0.1)  # d = 96
    Q = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dmu.DmuError):
        dmu.attention_bf16(Q, K, K, torch.empty_like(Q), 0.1, causal=True)  # Sq > Sk
    with pytest.raises(dmu.DmuError):
        dmu.attention_bf16(Q, Q, Q, torch.empty_like(Q), 0.0)  # scale
