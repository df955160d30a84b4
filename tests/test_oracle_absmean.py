"""Pins for the oracle's weight path: absmean gamma, ternarization, packing.

Sources: bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution",
section "The BitLinear Layer and AbsMean Quantization" (gamma = mean |W| of the
entire matrix; W / (gamma + eps), eps = 1e-5; round, clamp to [-1, 1]);
deepmox.com chapter 8, "A low-bit model is a whole-stack design" (values -1, 0,
+1; four ternary values per 8-bit storage unit).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle
from _exact import f32_bits, round_half_even, round_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def exact_absmean_f32(w):
    total = sum((Fraction(float(v)) for v in np.abs(w.astype(np.float64)).ravel()), Fraction(0))
    return round_to_f32(total / w.size)


# ---------------------------------------------------------------- gamma


@pytest.mark.parametrize("seed", range(6))
def test_absmean_matches_exact_rational_mean(seed):
    rng = np.random.default_rng(seed)
    n, k = rng.integers(1, 40), rng.integers(1, 90)
    w = (rng.standard_normal((n, k)) * 10.0 ** rng.uniform(-6, 3)).astype(np.float32)
    assert f32_bits(float(oracle.absmean(w))) == f32_bits(exact_absmean_f32(w))


def test_absmean_exact_where_fp32_summation_is_not():
    # one large value among many small ones: naive fp32 accumulation drops the small ones
    w = np.full(4097, 1.0, np.float32)
    w[0] = 2.0 ** 25
    got = float(oracle.absmean(w))
    assert f32_bits(got) == f32_bits(exact_absmean_f32(w))
    naive = np.float32(0)
    for v in w:
        naive = np.float32(naive + abs(v))
    assert float(naive / np.float32(w.size)) != got


def test_absmean_subnormal_and_mixed_binades():
    w = np.array([1e-45, -3e-44, 1e-40, 2.5e-39, -1e30, 7.0, -1e-20], np.float32)
    assert f32_bits(float(oracle.absmean(w))) == f32_bits(exact_absmean_f32(w))


def test_absmean_golden_cases():
    """Hand-worked cases (tests/golden/absmean_cases.json)."""
    with open(os.path.join(GOLDEN, "absmean_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        w = np.array([float.fromhex(v) for v in case["w"]], np.float32)
        want = float.fromhex(case["gamma"])
        got = float(oracle.absmean(w))
        assert got == want, case["why"]


def test_absmean_constant_magnitude():
    rng = np.random.default_rng(1)
    for c in (0.02, 1.0, 3.0e-30, 1.7e38):
        w = (np.float32(c) * np.where(rng.random((33, 65)) < 0.5, -1, 1)).astype(np.float32)
        assert oracle.absmean(w) == np.float32(c)


def test_absmean_zero_matrix():
    assert oracle.absmean(np.zeros((16, 64), np.float32)) == 0.0


def test_absmean_gaussian_closed_form():
    """E|W| = sigma * sqrt(2/pi) for W ~ N(0, sigma^2) (half-normal mean)."""
    sigma = 0.02
    w = datagen.weights(datagen.stream_id(1, 0, 0, datagen.TENSOR_W), 2560, 2560, sigma)
    g = float(oracle.absmean(w))
    expect = sigma * math.sqrt(2.0 / math.pi)
    # relative standard error sqrt(1 - 2/pi)/sqrt(2/pi)/sqrt(n) ~ 3e-4
    assert abs(g / expect - 1.0) < 2e-3


def test_absmean_independent_of_order_and_shape():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((48, 128)).astype(np.float32)
    g = oracle.absmean(w)
    assert oracle.absmean(w.T.copy()) == g
    assert oracle.absmean(rng.permutation(w.ravel())) == g


# ---------------------------------------------------------------- ternarize


def exact_ternarize(w, gamma):
    d = round_to_f32(Fraction(float(np.float32(gamma))) + Fraction(float(np.float32(1e-5))))
    out = []
    for v in w.ravel():
        r = round_to_f32(Fraction(float(v)) / Fraction(d))
        out.append(max(-1, min(1, round_half_even(Fraction(r)))))
    return np.array(out, np.int8).reshape(w.shape)


@pytest.mark.parametrize("seed", range(4))
def test_ternarize_matches_exact_rationals(seed):
    rng = np.random.default_rng(100 + seed)
    w = (rng.standard_normal((17, 70)) * 0.02).astype(np.float32)
    g = oracle.absmean(w)
    # put some elements exactly on the decision boundaries
    d = np.float32(np.float32(g) + np.float32(1e-5))
    w.ravel()[:6] = [d * np.float32(0.5), -d * np.float32(0.5), d * np.float32(1.5), d, -d, 0.0]
    np.testing.assert_array_equal(oracle.ternarize(w, g), exact_ternarize(w, g))


def test_ternarize_round_half_even_and_clamp():
    # gamma chosen so that gamma + 1e-5 rounds to exactly 1.0 in fp32
    gamma = np.float32(1.0) - np.float32(1e-5)
    assert np.float32(gamma + np.float32(1e-5)) == np.float32(1.0)
    w = np.array([0.5, -0.5, 0.50000006, -0.50000006, 1.5, 2.5, -2.5, 1e6, -1e6, 0.0, -0.0, 0.49999997],
                 np.float32)
    # round(0.5) = 0 and round(-0.5) = 0 (half to even); values past 1 clamp to +-1
    want = [0, 0, 1, -1, 1, 1, -1, 1, -1, 0, 0, 0]
    np.testing.assert_array_equal(oracle.ternarize(w, gamma), want)


def test_ternarize_threshold_invariant_and_trit_set():
    w = datagen.weights(datagen.stream_id(1, 0, 0, datagen.TENSOR_W), 512, 2560)
    g = oracle.absmean(w)
    q = oracle.ternarize(w, g)
    assert set(np.unique(q)) <= {-1, 0, 1}
    d = np.float32(g + np.float32(1e-5))
    r = (w / d).astype(np.float32)  # numpy fp32 division is IEEE, correctly rounded
    np.testing.assert_array_equal(q == 0, np.abs(r) <= 0.5)
    nz = q != 0
    np.testing.assert_array_equal(q[nz], np.sign(w[nz]).astype(np.int8))


def test_ternarize_zero_fraction_closed_form():
    """Zero trits occur where |z| <= 0.5 * sqrt(2/pi) (gamma ~ sigma sqrt(2/pi)):
    P = erf(0.5 * sqrt(2/pi) / sqrt(2)) ~ 0.3101."""
    w = datagen.weights(datagen.stream_id(1, 0, 0, datagen.TENSOR_W), 2560, 2560)
    q = oracle.ternarize(w, oracle.absmean(w))
    p = math.erf(0.5 * math.sqrt(2.0 / math.pi) / math.sqrt(2.0))
    assert abs((q == 0).mean() - p) < 2e-3
    assert abs((q == 1).mean() - (q == -1).mean()) < 2e-3


# ---------------------------------------------------------------- packing


def all_valid_bytes():
    out = []
    for a in range(3):
        for b in range(3):
            for c in range(3):
                for d in range(3):
                    out.append(a | (b << 2) | (c << 4) | (d << 6))
    return np.array(out, np.uint8)


def test_packed_size_is_four_trits_per_byte():
    for n, k in [(1, 64), (16, 64), (17, 128), (2560, 2560), (3, 6912)]:
        assert oracle.packed_bytes(n, k) == ((n + 15) // 16) * 16 * k // 4


def test_unpack_pack_roundtrip_over_all_81_byte_patterns():
    valid = all_valid_bytes()
    assert valid.size == 81  # 3^4 combinations of four trits
    rng = np.random.default_rng(3)
    n, k = 16 * 3, 64 * 5
    buf = rng.choice(valid, size=oracle.packed_bytes(n, k))
    buf[:81] = valid
    q = oracle.unpack(buf, n, k)
    assert set(np.unique(q)) <= {-1, 0, 1}
    np.testing.assert_array_equal(oracle.pack(q), buf)


@pytest.mark.parametrize("n,k", [(1, 64), (5, 128), (16, 64), (31, 192), (40, 2560)])
def test_pack_unpack_roundtrip(n, k):
    rng = np.random.default_rng(n * 1000 + k)
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    p = oracle.pack(q)
    np.testing.assert_array_equal(oracle.unpack(p, n, k), q)
    # padding rows of the last 16-row tile hold trit 0 (code 1)
    if n % 16:
        full = oracle.unpack(p, (n + 15) // 16 * 16, k)
        assert (full[n:] == 0).all()


def test_unpack_rejects_code_three():
    q = np.zeros((16, 64), np.int8)
    p = oracle.pack(q)
    for pos in (0, 100, p.size - 1):
        bad = p.copy()
        bad[pos] |= 0x30
        with pytest.raises(ValueError):
            oracle.unpack(bad, 16, 64)


def test_pack_single_trit_touches_one_two_bit_field():
    """Each trit owns exactly one 2-bit field of one byte, and the map from
    (row, column) to fields is one-to-one."""
    n, k = 20, 128
    base = oracle.pack(np.zeros((n, k), np.int8))
    assert (base == 0x55).all()
    seen = set()
    for row in range(n):
        for col in range(k):
            q = np.zeros((n, k), np.int8)
            q[row, col] = 1
            diff = np.nonzero(oracle.pack(q) != base)[0]
            assert diff.size == 1
            byte = int(diff[0])
            # code 1 -> code 2 in one field: the byte changes by 0b11 in that field only
            x = int(oracle.pack(q)[byte]) ^ 0x55
            assert x in (0x03, 0x0C, 0x30, 0xC0)
            seen.add((byte, x))
    assert len(seen) == n * k


def test_layout_fields_give_codes_in_column_order():
    """Documented property of the tiled layout: in row r of tile (i, j), the
    row's 16 bytes read as four little-endian 32-bit words v0..v3, shifted
    right by 2*f and masked with 0x03030303, hold the codes (trit + 1) of
    columns 64*j + 16*f + 4*w + 0..3 in word w, one per byte, in byte order;
    so field f of the 16 bytes is the 16 consecutive columns 64*j + 16*f + 0..15."""
    rng = np.random.default_rng(11)
    n, k = 35, 256
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    p = oracle.pack(q)
    words = p.view(np.uint32).reshape((n + 15) // 16, k // 64, 16, 4)  # [row tile][col tile][row][word]
    for ti in range((n + 15) // 16):
        for tj in range(k // 64):
            for r in range(16):
                row = ti * 16 + r
                for f in range(4):
                    codes = []
                    for wi in range(4):
                        codes += list(((int(words[ti, tj, r, wi]) >> (2 * f)) & 0x03030303).to_bytes(4, "little"))
                    cols = [64 * tj + 16 * f + b for b in range(16)]
                    want = [int(q[row, c]) + 1 if row < n else 1 for c in cols]
                    assert codes == want


def test_weight_path_end_to_end_small():
    """gamma, ternarize, pack and unpack composed, against the exact forms."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((19, 128)) * 0.02).astype(np.float32)
    packed, g = oracle.ternarize_pack(w)
    assert f32_bits(float(g)) == f32_bits(exact_absmean_f32(w))
    np.testing.assert_array_equal(oracle.unpack(packed, 19, 128), exact_ternarize(w, g))
