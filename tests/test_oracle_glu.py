"""Pins for the oracle's squared-ReLU gating after a fused gate+up BitLinear.

Sources: deepmox.com chapter 8, "A low-bit model is a whole-stack design", and
onilabs.co, "A Two-Billion Ternary Bet": the 2B4T feed-forward block uses
squared ReLU beside the ternary linear layers.  The pages print no formula;
the reading pinned here is the gated form h = relu(g)^2 * u, with g and u the
gate and up halves (rows 0..f-1 and f..2f-1) of one BitLinear with 2f output
rows and one gamma, evaluated exactly and rounded once to bf16.  The packed
form of such a matrix alternates 16-row tiles of gate and up rows.
"""
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle
from _exact import round_to_bf16_bits


def expected_glu_bits(acc_g: int, acc_u: int, gamma, alpha) -> int:
    s = Fraction(float(np.float32(gamma))) * Fraction(float(np.float32(alpha))) / 127
    g, u = acc_g * s, acc_u * s
    r = max(g, Fraction(0))
    exact = r * r * u
    if exact == 0:  # IEEE: (+0) * negative u is -0
        return 0x8000 if u < 0 else 0
    return round_to_bf16_bits(exact)


@pytest.mark.parametrize("seed", range(4))
def test_glu_matches_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    m, f = 3, 40
    acc = rng.integers(-200_000, 200_000, size=(m, 2 * f)).astype(np.int32)
    acc[0, :4] = [0, -1, 1, 5]
    acc[0, f:f + 4] = [-3, -3, 0, -7]
    gamma = np.float32(rng.uniform(0.001, 0.05))
    alpha = datagen.bf16_to_f32(datagen.f32_to_bf16(rng.uniform(0.5, 80, size=m).astype(np.float32)))
    h = oracle.glu(acc, gamma, alpha)
    assert h.shape == (m, f)
    for i in range(m):
        for j in range(f):
            assert int(h[i, j]) == expected_glu_bits(int(acc[i, j]), int(acc[i, f + j]), gamma, alpha[i]), (i, j)


def test_glu_worked_example():
    # acc_g = 254, acc_u = -127, gamma = 0.5, alpha = 127: s = 0.5, g = 127,
    # u = -63.5, h = 127^2 * -63.5 = -1024191.5.  Near 2^19.97 the bf16 spacing
    # is 2^12 = 4096; 1024191.5 / 4096 = 250.05 -> 250 * 4096 = 1024000 =
    # 1.953125 * 2^19: sign 1, exponent 127 + 19 = 0x92, mantissa 0x7A -> 0xC97A.
    h = oracle.glu(np.array([[254, -127]], np.int32), 0.5, np.array([127.0], np.float32))
    assert int(h[0, 0]) == 0xC97A


def test_glu_unit_scale_integers():
    # gamma = 127, alpha = 1: s = 1, so g and u are the accumulators themselves
    cases = [
        (3, 5, 0x4234),      # 9 * 5 = 45 = 1.40625 * 2^5, exact
        (16, 1, 0x4380),     # 256
        (17, 1, 0x4390),     # 289 is halfway between 288 and 290: ties to even -> 288
        (-4, 9, 0x0000),     # gate below zero: relu gives +0
        (-4, -9, 0x8000),    # +0 times a negative up value is -0
        (0, -1, 0x8000),
        (7, 0, 0x0000),      # up value zero
        (-2, 3, 0x0000),
    ]
    acc = np.array([[g for g, _, _ in cases] + [u for _, u, _ in cases]], np.int32)
    h = oracle.glu(acc, 127.0, np.array([1.0], np.float32))
    assert [int(v) for v in h[0]] == [bits for _, _, bits in cases]


def test_pack_glu_alternates_gate_and_up_tiles():
    rng = np.random.default_rng(5)
    f, k = 48, 128
    q = rng.integers(-1, 2, size=(2 * f, k)).astype(np.int8)
    packed = oracle.pack_glu(q)
    assert packed.size == oracle.packed_bytes(2 * f, k)
    plain = oracle.unpack(packed, 2 * f, k)  # rows in packed order
    order = []
    for t in range(f // 16):
        order += list(range(16 * t, 16 * t + 16))            # gate tile t
        order += list(range(f + 16 * t, f + 16 * t + 16))    # up tile t
    np.testing.assert_array_equal(plain, q[order])
    np.testing.assert_array_equal(oracle.unpack_glu(packed, f, k), q)
    # the alternating packing is the plain packing of the reordered rows
    np.testing.assert_array_equal(packed, oracle.pack(q[order]))


def test_pack_glu_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.pack_glu(np.zeros((2 * 24, 64), np.int8))   # f not a multiple of 16
    with pytest.raises(ValueError):
        oracle.pack_glu(np.zeros((32, 96), np.int8))       # k not a multiple of 64


def test_glu_forward_composes_the_steps():
    f, k, m = 32, 320, 3
    w = datagen.weights(datagen.stream_id(1, 0, 2, 0), 2 * f, k)
    packed, g = oracle.ternarize_pack_glu(w)
    assert g == oracle.absmean(w)
    qw = oracle.ternarize(w, g)
    np.testing.assert_array_equal(oracle.unpack_glu(packed, f, k), qw)
    x = datagen.activations_bf16(datagen.stream_id(1, 0, 2, 1), m, k)
    h, acc, xq, alpha = oracle.bitlinear_glu_forward(packed, g, x, f)
    qx, a = oracle.quant_act(x)
    np.testing.assert_array_equal(xq, qx)
    np.testing.assert_array_equal(alpha, a)
    np.testing.assert_array_equal(acc, oracle.linear_mul(qw, qx))
    np.testing.assert_array_equal(h, oracle.glu(acc, g, a))
    # loose sanity against the unquantized layer: relu(x Wg)^2 * (x Wu)
    xf = datagen.bf16_to_f32(x).reshape(m, k).astype(np.float64)
    wd = qw.astype(np.float64) * float(g)
    gate, up = xf @ wd[:f].T, xf @ wd[f:].T
    ref = np.maximum(gate, 0) ** 2 * up
    got = datagen.bf16_to_f32(h).reshape(m, f)
    assert np.abs(got - ref).max() <= 0.1 * np.abs(ref).max()
