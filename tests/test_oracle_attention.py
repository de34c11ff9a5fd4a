"""Pins for the oracle's attention chain, O = softmax(scale * Q K^T) V per head
(the two-product chain with an elementwise step between the products that the
"Tensor Cores" chapter (ai-infra-handbooks), section "mma.sync: the register
layout is explicit", names as FlashAttention's case).

Independent references: numpy matmuls with scipy's softmax and logsumexp on
an explicitly built mask; closed forms (constant V, identical keys, zero
scale, a single key, the first causal row); the permutation symmetry of
(K, V); and the sign structure of Aabs."""
import numpy as np
import pytest
import scipy.special as sp

import oracle
from dense_matrix_unit_amd import workloads as wl


def bf16(shape, seed, mult=1.0):
    return oracle.encode_bf16((wl.normal(shape, seed) * np.float32(mult)).astype(np.float32))


def reference(Q, K, V, scale, causal):
    """numpy / scipy: scores by matmul, masked by np.tril, softmax and
    logsumexp from scipy."""
    q, k, v = (oracle.decode_bf16(x) for x in (Q, K, V))
    S = scale * (q @ np.swapaxes(k, -1, -2))
    Sq, Sk = S.shape[-2:]
    if causal:
        allowed = np.tril(np.ones((Sq, Sk), bool), k=Sk - Sq)
        S = np.where(allowed, S, -np.inf)
    P = sp.softmax(S, axis=-1)
    return P @ v, sp.logsumexp(S, axis=-1), P @ np.abs(v)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 7, 9, 16), (3, 33, 65, 64), (2, 40, 40, 128)])
def test_matches_numpy_scipy(shape, causal):
    BH, Sq, Sk, d = shape
    Q, K, V = bf16((BH, Sq, d), 1), bf16((BH, Sk, d), 2), bf16((BH, Sk, d), 3)
    scale = 1.0 / np.sqrt(d)
    O, lse, A = oracle.attention_bf16(Q, K, V, scale, causal)
    Or, lr, Ar = reference(Q, K, V, scale, causal)
    np.testing.assert_allclose(O, Or, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lr, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(A, Ar, rtol=1e-12, atol=1e-13)


def test_constant_values_give_that_constant():
    # every weight vector sums to one, so V = c everywhere gives O = c
    Q, K = bf16((4, 50, 32), 4, 3.0), bf16((4, 70, 32), 5, 3.0)
    V = np.full((4, 70, 32), oracle.encode_bf16(np.float32([-2.5]))[0], np.uint16)
    for causal in (False, True):
        O, _, A = oracle.attention_bf16(Q, K, V, 0.7, causal)
        np.testing.assert_allclose(O, -2.5, rtol=1e-14)
        np.testing.assert_allclose(A, 2.5, rtol=1e-14)


def test_identical_keys_or_zero_scale_average_the_values():
    Q, V = bf16((2, 9, 16), 6), bf16((2, 12, 16), 7)
    K = np.repeat(bf16((2, 1, 16), 8), 12, axis=1)
    v = oracle.decode_bf16(V)
    O, lse, _ = oracle.attention_bf16(Q, K, V, 0.25)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=1, keepdims=True), O.shape),
                               rtol=1e-13, atol=1e-14)
    # equal scores: lse = s + log(Sk)
    s = 0.25 * np.einsum("bid,bd->bi", oracle.decode_bf16(Q), oracle.decode_bf16(K[:, 0]))
    np.testing.assert_allclose(lse, s + np.log(12), rtol=1e-13, atol=1e-13)
    # zero scale with the causal mask: row i averages keys 0 .. i + Sk - Sq
    K2 = bf16((2, 12, 16), 9)
    O, lse, _ = oracle.attention_bf16(Q, K2, V, 0.0, causal=True)
    for i in range(9):
        n = i + 12 - 9 + 1
        np.testing.assert_allclose(O[:, i], v[:, :n].mean(axis=1), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, i], np.log(n), rtol=1e-14)


def test_single_visible_key_returns_its_value_exactly():
    Q, K, V = bf16((3, 5, 8), 10), bf16((3, 1, 8), 11), bf16((3, 1, 8), 12)
    O, _, _ = oracle.attention_bf16(Q, K, V, 0.9)
    assert np.array_equal(O, np.broadcast_to(oracle.decode_bf16(V), O.shape))
    # causal with Sq == Sk: row 0 sees key 0 only
    Q, K, V = bf16((2, 6, 8), 13), bf16((2, 6, 8), 14), bf16((2, 6, 8), 15)
    O, lse, _ = oracle.attention_bf16(Q, K, V, 0.5, causal=True)
    assert np.array_equal(O[:, 0], oracle.decode_bf16(V[:, 0]))
    q0k0 = np.sum(oracle.decode_bf16(Q[:, 0]) * oracle.decode_bf16(K[:, 0]), axis=-1)
    np.testing.assert_allclose(lse[:, 0], 0.5 * q0k0, rtol=1e-15)


def test_permuting_keys_with_their_values_changes_nothing():
    Q, K, V = bf16((2, 11, 32), 16), bf16((2, 37, 32), 17), bf16((2, 37, 32), 18)
    perm = np.random.default_rng(0).permutation(37)
    O1, l1, _ = oracle.attention_bf16(Q, K, V, 0.2)
    O2, l2, _ = oracle.attention_bf16(Q, K[:, perm], V[:, perm], 0.2)
    np.testing.assert_allclose(O1, O2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


def test_aabs_bounds_o_and_equals_it_for_nonnegative_values():
    Q, K, V = bf16((2, 20, 16), 19), bf16((2, 30, 16), 20), bf16((2, 30, 16), 21)
    O, _, A = oracle.attention_bf16(Q, K, V, 0.4)
    assert np.all(np.abs(O) <= A * (1 + 1e-14))
    Vp = oracle.encode_bf16(np.abs(oracle.decode_bf16(V)).astype(np.float32))
    O, _, A = oracle.attention_bf16(Q, K, Vp, 0.4)
    np.testing.assert_allclose(O, A, rtol=1e-14)


def test_large_scores_do_not_overflow():
    # scores of several thousand: the max subtraction keeps exp finite
    Q, K, V = bf16((1, 8, 64), 22, 30.0), bf16((1, 16, 64), 23, 30.0), bf16((1, 16, 64), 24)
    O, lse, _ = oracle.attention_bf16(Q, K, V, 1.0)
    Or, lr, _ = reference(Q, K, V, 1.0, False)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(O, Or, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lr, rtol=1e-13)


def test_argument_errors():
    Q = bf16((1, 5, 8), 25)
    K = bf16((1, 4, 8), 26)
    with pytest.raises(ValueError):
        oracle.attention_bf16(Q, K, K, 1.0, causal=True)  # Sq > Sk
