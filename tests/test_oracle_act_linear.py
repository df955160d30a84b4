"""Pins for the oracle's activation quantizer, integer product and rescale.

Sources: deepmox.com chapter 8, "A low-bit model is a whole-stack design"
(activations take a separate per-token 8-bit path; W1.58A8); onilabs.co, "A
Two-Billion Ternary Bet" (activations are quantized dynamically); bako.co,
"The BitLinear Layer and AbsMean Quantization" (with weights in {-1, 0, 1} the
product needs only additions and subtractions).  The scale 127 / absmax and
the output y = acc * gamma * absmax / 127 in bf16 are the plainest reading of
"per-token 8-bit" with an absmax scale; the pages print no numeric example.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
import oracle
from _exact import bf16_value, round_half_even, round_to_bf16_bits, round_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(values):
    return datagen.f32_to_bf16(np.asarray(values, np.float32))


# ---------------------------------------------------------------- quantizer


def exact_quant_row(bits_row):
    xs = [bf16_value(int(b)) for b in bits_row]
    amax = max(abs(v) for v in xs)
    s = round_to_f32(Fraction(127) / max(amax, Fraction(float(np.float32(1e-5)))))
    q = []
    for v in xs:
        prod = round_to_f32(v * Fraction(s))
        q.append(max(-128, min(127, round_half_even(Fraction(prod)))))
    return q, float(amax)


@pytest.mark.parametrize("seed", range(5))
def test_quant_matches_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    m, k = 3, 96
    x = bf16_bits(rng.standard_normal((m, k)) * 10.0 ** rng.uniform(-3, 3))
    q, a = oracle.quant_act(x)
    for i in range(m):
        want_q, want_a = exact_quant_row(x[i])
        assert list(q[i]) == want_q
        assert float(a[i]) == want_a


def test_quant_golden_ties():
    """Hand-worked rows (tests/golden/quant_cases.json)."""
    with open(os.path.join(GOLDEN, "quant_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        x = bf16_bits([float(v) for v in case["x"]])[None, :]
        q, a = oracle.quant_act(x)
        assert list(q[0]) == case["q"], case["why"]
        assert float(a[0]) == case["alpha"], case["why"]


def test_quant_invariants_on_workload_rows():
    k = 2560
    cols = datagen.outlier_columns(datagen.WORKLOAD_STACK_2B, k, datagen.STACK_2B_OUTLIERS)
    x = datagen.activations_bf16(datagen.stream_id(2, 0, 0, 1), 64, k, cols, 20.0)
    q, a = oracle.quant_act(x)
    xf = datagen.bf16_to_f32(x).reshape(64, k).astype(np.float64)
    amax = np.abs(xf).max(axis=1)
    np.testing.assert_array_equal(a, amax.astype(np.float32))
    assert np.abs(q).max() <= 127
    for i in range(64):
        j = int(np.argmax(np.abs(xf[i])))
        assert abs(int(q[i, j])) == 127
    # sign agreement and the quantization error bound |x - q*amax/127| <= amax/254 (+ fp32 slack)
    assert ((np.sign(q) == np.sign(xf)) | (q == 0)).all()
    err = np.abs(xf - q * (amax[:, None] / 127.0))
    assert (err <= amax[:, None] / 254.0 * (1 + 1e-6)).all()
    # outlier channels dominate the absmax
    assert (np.abs(xf[:, cols]).max(axis=1) == amax).mean() > 0.9


def test_quant_odd_symmetry_and_row_independence():
    rng = np.random.default_rng(9)
    x = bf16_bits(rng.standard_normal((5, 128)))
    q, a = oracle.quant_act(x)
    qn, an = oracle.quant_act(x ^ np.uint16(0x8000))
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(an, a)
    perm = np.array([3, 0, 4, 1, 2])
    qp, ap = oracle.quant_act(x[perm])
    np.testing.assert_array_equal(qp, q[perm])
    np.testing.assert_array_equal(ap, a[perm])


def test_quant_zero_row():
    q, a = oracle.quant_act(np.zeros((2, 64), np.uint16))
    assert (q == 0).all() and (a == 0).all()


# ---------------------------------------------------------------- integer product


def bigint_product(qw, qx):
    m, k = qx.shape
    n = qw.shape[0]
    return [[sum(int(qx[i, t]) * int(qw[j, t]) for t in range(k)) for j in range(n)] for i in range(m)]


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (1, 7, 64), (3, 5, 130), (17, 9, 64), (2, 31, 200)])
def test_linear_brute_force(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    qw = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    qx = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    acc = oracle.linear_mul(qw, qx)
    assert acc.tolist() == bigint_product(qw, qx)
    ref = torch.from_numpy(qx).long() @ torch.from_numpy(qw).long().T
    np.testing.assert_array_equal(acc, ref.numpy())
    np.testing.assert_array_equal(oracle.linear_add(qw, qx), acc)


def test_linear_addition_only_form_equals_product_on_workload():
    w = datagen.weights(datagen.stream_id(1, 0, 0, 0), 256, 2560)
    qw = oracle.ternarize(w, oracle.absmean(w))
    x = datagen.activations_bf16(datagen.stream_id(1, 0, 0, 1), 4, 2560)
    qx, _ = oracle.quant_act(x)
    np.testing.assert_array_equal(oracle.linear_add(qw, qx), oracle.linear_mul(qw, qx))


def test_linear_extremes_and_linearity():
    k = 6912
    qw = np.ones((3, k), np.int8)
    qw[1] = -1
    qw[2, ::2] = 0
    qx = np.full((2, k), 127, np.int8)
    qx[1] = -127
    acc = oracle.linear_mul(qw, qx)
    assert acc.tolist() == [[127 * k, -127 * k, 127 * k // 2], [-127 * k, 127 * k, -127 * k // 2]]
    rng = np.random.default_rng(2)
    qw = rng.integers(-1, 2, size=(8, 256)).astype(np.int8)
    qx = rng.integers(-127, 128, size=(3, 256)).astype(np.int8)
    np.testing.assert_array_equal(oracle.linear_mul(qw, -qx), -oracle.linear_mul(qw, qx))


# ---------------------------------------------------------------- rescale


def test_bf16_rounding_golden():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2 ** -8, 0x3F80),           # halfway 1 / 1+2^-7: ties to even (1)
        (1.0 + 3 * 2 ** -8, 0x3F82),       # halfway 1+2^-7 / 1+2^-6: ties to even (1+2^-6)
        (1.0 + 2 ** -8 + 2 ** -40, 0x3F81),  # just past halfway
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (2.0 ** -133, 0x0001),             # smallest bf16 subnormal
        (2.0 ** -134, 0x0000),             # halfway 0 / 2^-133: ties to 0
        (3.3895313892515355e38, 0x7F7F),   # largest finite bf16
        (3.4e38, 0x7F80),                  # rounds past the largest finite value
    ]
    for v, bits in cases:
        assert oracle.bf16_from_double(v) == bits, v


@pytest.mark.parametrize("seed", range(4))
def test_rescale_matches_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    m, n = 3, 50
    acc = rng.integers(-3_000_000, 3_000_000, size=(m, n)).astype(np.int32)
    acc[0, :3] = [0, 1, -1]
    gamma = np.float32(rng.uniform(0.001, 0.05))
    alpha = datagen.bf16_to_f32(bf16_bits(rng.uniform(0.5, 80, size=m)))
    y = oracle.rescale(acc, gamma, alpha)
    for i in range(m):
        for j in range(n):
            exact = Fraction(int(acc[i, j])) * Fraction(float(gamma)) * Fraction(float(alpha[i])) / 127
            assert int(y[i, j]) == round_to_bf16_bits(exact)
    assert (y[0, 0] == 0)


def test_forward_composes_the_steps():
    w = datagen.weights(datagen.stream_id(1, 0, 0, 0), 40, 256)
    packed, g = oracle.ternarize_pack(w)
    x = datagen.activations_bf16(datagen.stream_id(1, 0, 0, 1), 3, 256)
    y, acc, xq, alpha = oracle.bitlinear_forward(packed, g, x, 40)
    qx, a = oracle.quant_act(x)
    np.testing.assert_array_equal(xq, qx)
    np.testing.assert_array_equal(alpha, a)
    qw = oracle.unpack(packed, 40, 256)
    np.testing.assert_array_equal(acc, oracle.linear_mul(qw, qx))
    np.testing.assert_array_equal(y, oracle.rescale(acc, g, a))
    # loose sanity against the unquantized product: relative error of a ternary layer
    ref = datagen.bf16_to_f32(x).reshape(3, 256).astype(np.float64) @ (qw.astype(np.float64) * float(g)).T
    got = datagen.bf16_to_f32(y).reshape(3, 40)
    assert np.abs(got - ref).max() <= 0.05 * np.abs(ref).max()


# ---------------------------------------------------------------- input generator


def test_datagen_is_deterministic_and_standard_normal():
    a = datagen.normal_f32(12345, 1 << 20)
    b = datagen.normal_f32(12345, 1 << 20)
    np.testing.assert_array_equal(a, b)
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1) < 5e-3
    assert abs(np.abs(a).mean() - np.sqrt(2 / np.pi)) < 5e-3
    c = datagen.normal_f32(12346, 1 << 10)
    assert not np.array_equal(a[: 1 << 10], c)


def test_datagen_outlier_columns():
    cols = datagen.outlier_columns(datagen.WORKLOAD_70B, 28672, datagen.n_outliers_70b(28672))
    assert cols.size == 29 and np.unique(cols).size == 29
    assert datagen.n_outliers_70b(8192) == 8
    x = datagen.activations_bf16(77, 2, 28672, cols, 30.0)
    xf = np.abs(datagen.bf16_to_f32(x).reshape(2, 28672))
    assert xf[:, cols].mean() > 20 * np.delete(xf, cols, axis=1).mean()
