"""Pins for the oracle's straight-through backward of the BitLinear.

Source: bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution",
section "Training Dynamics: The Straight-Through Estimator": the backward pass
treats the rounding step as the identity; gradients reach high-precision
shadow weights.  Reading pinned here: both quantizers are the identity in the
backward pass and their scales are constants, so for the dequantized forward
y = xhat What^T (xhat = alpha/127 qx, What = gamma q):
    dx = gamma * dy q,     dw = dy^T (alpha/127 qx),
evaluated exactly and rounded once to fp32.  The pins are exact rationals, the
adjoint identities of the linear map (which fail for a transposed or
misplaced operand), special values, and the transposed packing.
"""
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle
from _exact import bf16_value, round_to_f32


def f32_ulp(v: float) -> float:
    a = abs(np.float32(v))
    return float(np.spacing(a)) if a > 0 else float(np.spacing(np.float32(0)))


def random_dy(rng, m, n, scale=1.0):
    return datagen.f32_to_bf16((rng.standard_normal((m, n)) * scale).astype(np.float32))


@pytest.mark.parametrize("seed", range(3))
def test_backward_x_matches_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    m, n, k = 2, 40, 128
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    packed = oracle.pack(q)
    gamma = np.float32(rng.uniform(0.005, 0.05))
    dy = random_dy(rng, m, n)
    dx = oracle.backward_x(packed, gamma, dy, n, k)
    for i in range(m):
        for t in range(0, k, 7):
            exact = Fraction(float(gamma)) * sum(bf16_value(int(dy[i, j])) * int(q[j, t]) for j in range(n))
            want = round_to_f32(exact)
            assert abs(float(dx[i, t]) - want) <= f32_ulp(want), (i, t)


@pytest.mark.parametrize("seed", range(3))
def test_backward_w_matches_exact_rationals(seed):
    rng = np.random.default_rng(10 + seed)
    m, n, k = 5, 12, 64
    dy = random_dy(rng, m, n)
    qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    alpha = datagen.bf16_to_f32(datagen.f32_to_bf16(rng.uniform(0.5, 30, size=m).astype(np.float32)))
    dw = oracle.backward_w(dy, qx, alpha)
    for j in range(n):
        for t in range(0, k, 5):
            exact = sum(bf16_value(int(dy[i, j])) * Fraction(float(alpha[i])) * int(qx[i, t]) for i in range(m)) / 127
            assert float(dw[j, t]) == round_to_f32(exact), (j, t)


def test_backward_adjoint_identities():
    """<dy, x dW^T> = <dw, dW> and <dy, dx What^T> = <dx_grad, dx> for the
    dequantized linear map; exact in binary64 up to rounding of the oracle's
    fp32 outputs."""
    rng = np.random.default_rng(3)
    m, n, k = 4, 48, 192
    w = datagen.weights(7, n, k)
    packed, gamma = oracle.ternarize_pack(w)
    q = oracle.unpack(packed, n, k).astype(np.float64)
    x = datagen.activations_bf16(8, m, k)
    qx, alpha = oracle.quant_act(x)
    xhat = alpha.astype(np.float64)[:, None] / 127 * qx.astype(np.float64)
    what = float(gamma) * q
    dy = random_dy(rng, m, n)
    dyf = datagen.bf16_to_f32(dy).reshape(m, n).astype(np.float64)
    # input direction
    dx = oracle.backward_x(packed, gamma, dy, n, k).astype(np.float64)
    delta_x = rng.standard_normal((m, k))
    lhs = np.sum(dyf * (delta_x @ what.T))
    rhs = np.sum(dx * delta_x)
    assert abs(lhs - rhs) <= 1e-6 * np.sum(np.abs(dyf) @ np.abs(what) * np.abs(delta_x))
    # weight direction
    dw = oracle.backward_w(dy, qx, alpha).astype(np.float64)
    delta_w = rng.standard_normal((n, k))
    lhs = np.sum(dyf * (xhat @ delta_w.T))
    rhs = np.sum(dw * delta_w)
    assert abs(lhs - rhs) <= 1e-6 * np.sum(np.abs(dyf).T @ np.abs(xhat) * np.abs(delta_w))


def test_backward_special_values():
    rng = np.random.default_rng(4)
    m, n, k = 3, 16, 64
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    packed = oracle.pack(q)
    dy = random_dy(rng, m, n)
    assert not oracle.backward_x(packed, 0.0, dy, n, k).any()
    assert not oracle.backward_x(packed, 0.5, np.zeros((m, n), np.uint16), n, k).any()
    # gamma = 1, one nonzero gradient entry: dx is that entry times the row of q
    one = datagen.f32_to_bf16(np.zeros((1, n), np.float32))
    one[0, 5] = datagen.f32_to_bf16(np.array([2.0], np.float32))[0]
    dx = oracle.backward_x(packed, 1.0, one, n, k)
    np.testing.assert_array_equal(dx[0], 2.0 * q[5].astype(np.float32))
    qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    assert not oracle.backward_w(dy, qx, np.zeros(m, np.float32)).any()
    # alpha = 127, one token: dw is the outer product dy^T qx
    dw = oracle.backward_w(dy[:1], qx[:1], np.array([127.0], np.float32))
    want = datagen.bf16_to_f32(dy[:1]).reshape(1, n).astype(np.float64).T @ qx[:1].astype(np.float64)
    np.testing.assert_array_equal(dw, want.astype(np.float32))


def test_pack_transposed():
    rng = np.random.default_rng(5)
    n, k = 128, 192
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    packed = oracle.pack(q)
    packed_t = oracle.pack_transposed(packed, n, k)
    assert packed_t.size == oracle.packed_bytes(k, n)
    np.testing.assert_array_equal(oracle.unpack(packed_t, k, n), q.T)
    with pytest.raises(ValueError):
        oracle.pack_transposed(oracle.pack(q[:96]), 96, k)  # n must be a multiple of 64
