"""Pins for the oracle's fused epilogue, Y = act(alpha * D + bias) ("How
Blackwell's Tensor Memory Actually Works", section "The cost of getting the
answer back": scale, bias, activation, cast down).  References: numpy for the
affine part, scipy's erf and logistic function, closed forms and the odd-part
identities act(x) - act(-x) = x of GELU and SiLU."""
import numpy as np
import scipy.special as sp

import oracle
from dense_matrix_unit_amd import workloads as wl


def test_affine_part():
    D = wl.normal((7, 33), 1).astype(np.float64)
    b = wl.normal((33,), 2)
    Y = oracle.epilogue(D, 0.375, b)
    assert np.array_equal(Y, 0.375 * D + b.astype(np.float64))
    assert np.array_equal(oracle.epilogue(D), D)


def test_relu():
    D = np.array([[-2.0, -0.0, 0.0, 3.5, np.nan, -np.inf, np.inf]])
    Y = oracle.epilogue(D, act=oracle.ACT_RELU)
    assert Y.tolist()[0][:4] == [0.0, 0.0, 0.0, 3.5]
    assert Y[0, 4] == 0.0 and Y[0, 5] == 0.0 and Y[0, 6] == np.inf


def test_gelu_closed_forms_and_scipy():
    x = np.linspace(-9, 9, 721).reshape(1, -1)
    Y = oracle.epilogue(x, act=oracle.ACT_GELU)
    ref = x * 0.5 * (1 + sp.erf(x / np.sqrt(2)))
    # 1 + erf(x / sqrt 2) cancels to 0 or one ulp far in the negative tail
    assert np.allclose(Y, ref, rtol=1e-15, atol=1e-14)
    # Phi(1) = (1 + erf(1/sqrt 2)) / 2, erf(1/sqrt 2) = 0.6826894921370859 (the
    # one-sigma mass of the normal distribution)
    assert abs(oracle.epilogue(np.array([[1.0]]), act=2)[0, 0] - 0.8413447460685429) < 1e-15
    # x Phi(x) - (-x) Phi(-x) = x (Phi(x) + Phi(-x) = 1)
    Yn = oracle.epilogue(-x, act=oracle.ACT_GELU)
    assert np.allclose(Y - Yn, x, rtol=0, atol=1e-14)
    assert oracle.epilogue(np.array([[0.0]]), act=2)[0, 0] == 0.0


def test_silu_closed_forms_and_scipy():
    x = np.linspace(-30, 30, 1201).reshape(1, -1)
    Y = oracle.epilogue(x, act=oracle.ACT_SILU)
    assert np.allclose(Y, x * sp.expit(x), rtol=1e-14, atol=1e-300)
    assert abs(oracle.epilogue(np.array([[1.0]]), act=3)[0, 0] - 1 / (1 + np.exp(-1.0))) < 1e-16
    Yn = oracle.epilogue(-x, act=oracle.ACT_SILU)
    assert np.allclose(Y - Yn, x, rtol=0, atol=1e-13)
    assert oracle.epilogue(np.array([[-800.0]]), act=3)[0, 0] == 0.0   # exp overflow -> -0


def test_bias_then_activation_order():
    D = np.array([[-1.0, 1.0]])
    b = np.float32([2.0, -3.0])
    Y = oracle.epilogue(D, 1.0, b, act=oracle.ACT_RELU)
    assert Y.tolist() == [[1.0, 0.0]]
