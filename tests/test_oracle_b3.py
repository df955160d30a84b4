"""Pins for the oracle's five-trits-per-byte weight code.

Sources: bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution",
section "The Information Theory of 1.58 Bits" (a three-state weight carries
log2(3), about 1.58, bits); deepmox.com chapter 1, "Why Smaller Weights Are
Not the Whole Story", section "A different place to make efficiency
decisions" (the 2B4T model's non-embedding weights take 0.4 GB, less than two
bits per weight).  The format is a reading (the pages give none): five trits
per byte as the base-3 value v = sum_d (t_d + 1) 3^(4-d), stored as
ceil(256 v / 243); 16-row x 320-column super-tiles of 1024 bytes.
"""
import itertools
import json
import os

import numpy as np
import pytest

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALL5 = [np.array(t, np.int8) for t in itertools.product((-1, 0, 1), repeat=5)]


def test_every_five_trit_pattern_round_trips_to_a_distinct_byte():
    bytes_ = [oracle.b3_encode(t) for t in ALL5]
    assert len(set(bytes_)) == 243  # 3^5 patterns, one byte each
    assert all(0 <= b <= 255 for b in bytes_)
    for t, b in zip(ALL5, bytes_):
        np.testing.assert_array_equal(oracle.b3_decode(b), t)
    # order: the byte grows with the base-3 value (t_0 most significant)
    values = [sum(int(c + 1) * 3 ** (4 - d) for d, c in enumerate(t)) for t in ALL5]
    order = np.argsort(values)
    assert all(bytes_[order[i]] < bytes_[order[i + 1]] for i in range(242))
    # the 13 bytes that encode nothing are rejected
    others = sorted(set(range(256)) - set(bytes_))
    assert len(others) == 13
    assert all(oracle.b3_decode(b) is None for b in others)


def test_golden_bytes():
    """Hand-worked encodings (tests/golden/b3_cases.json)."""
    with open(os.path.join(GOLDEN, "b3_cases.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        assert oracle.b3_encode(case["trits"]) == case["byte"], case["why"]
        np.testing.assert_array_equal(oracle.b3_decode(case["byte"]), case["trits"])
    for b in data["not_codes"]:
        assert oracle.b3_decode(b) is None, data["not_codes_why"]


def test_every_code_also_decodes_by_multiply_and_carry():
    """The byte read as the base-3 fraction b / 256: digit d is the carry out
    of the low byte when (b * 3^d mod 256) is multiplied by 3.  This route
    needs no division; it holds for every code because rounding up keeps
    b / 256 within [v / 243, (v + 1) / 243)."""
    for t in ALL5:
        b = oracle.b3_encode(t)
        p = b
        for d in range(5):
            prod = p * 3
            assert prod >> 8 == int(t[d]) + 1
            p = prod & 0xFF


def test_sizes():
    assert oracle.packed_bytes_b3(16, 320) == 1024
    assert oracle.packed_bytes_b3(17, 64) == 32 * 64
    # rows of 2560 columns: exactly 1.6 bits per weight, 20% under the 2-bit code
    assert oracle.packed_bytes_b3(2560, 2560) * 5 == 2560 * 2560
    assert oracle.packed_bytes_b3(2560, 2560) / oracle.packed_bytes(2560, 2560) == 0.8
    # the 70B shapes (the last super-tile of a row is partial)
    assert oracle.packed_bytes_b3(57344, 8192) == 57344 * 26 * 64
    assert oracle.packed_bytes_b3(8192, 28672) == 8192 * 90 * 64


def super_tile_digits(buf, band, s, g, r, d, supers):
    """Digit d of the 16 bytes of group g, row r of super-tile (band, s),
    decoded by the multiply-and-carry route."""
    base = (band * supers + s) * 1024 + g * 256 + r * 16
    out = []
    for j in range(16):
        p = int(buf[base + j])
        for _ in range(d):
            p = (p * 3) & 0xFF
        out.append(((p * 3) >> 8) - 1)
    return np.array(out, np.int8)


@pytest.mark.parametrize("n,k", [(16, 320), (33, 640), (20, 192), (5, 1088)])
def test_documented_digit_column_property(n, k):
    """Digit d of the 16 bytes that group g of row r owns in super-tile s is
    columns 320 s + 80 g + 16 d .. + 15 of that row: read back from random
    trits through the property a decoder relies on, padding included."""
    rng = np.random.default_rng(n * 1000 + k)
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    buf = oracle.pack_b3(q)
    supers = (k + 319) // 320
    n_pad = (n + 15) // 16 * 16
    q_pad = np.zeros((n_pad, supers * 320), np.int8)
    q_pad[:n, :k] = q
    for band in range(n_pad // 16):
        for s in range(supers):
            for g in range(4):
                for r in range(16):
                    for d in range(5):
                        c0 = 320 * s + 80 * g + 16 * d
                        np.testing.assert_array_equal(super_tile_digits(buf, band, s, g, r, d, supers),
                                                      q_pad[16 * band + r, c0:c0 + 16])


@pytest.mark.parametrize("n,k", [(1, 64), (16, 320), (17, 384), (40, 2560), (9, 6912), (3, 8192)])
def test_round_trip_and_agreement_with_the_2bit_code(n, k):
    rng = np.random.default_rng(n + 7 * k)
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    buf = oracle.pack_b3(q)
    assert buf.size == oracle.packed_bytes_b3(n, k)
    np.testing.assert_array_equal(oracle.unpack_b3(buf, n, k), q)
    np.testing.assert_array_equal(oracle.unpack_b3(buf, n, k), oracle.unpack(oracle.pack(q), n, k))


def test_single_trit_changes_one_byte():
    """One nonzero trit against an all-zero matrix changes exactly one byte,
    in one digit; distinct positions use distinct (byte, digit) slots."""
    n, k = 32, 704
    zero = oracle.pack_b3(np.zeros((n, k), np.int8))
    assert (zero == 128).all()  # all-zero five-trit groups
    owner = {}
    rng = np.random.default_rng(3)
    for _ in range(300):
        row, col = int(rng.integers(n)), int(rng.integers(k))
        q = np.zeros((n, k), np.int8)
        q[row, col] = 1
        buf = oracle.pack_b3(q)
        diff = np.nonzero(buf != zero)[0]
        assert diff.size == 1
        t = oracle.b3_decode(buf[diff[0]])
        assert (t != 0).sum() == 1 and t.sum() == 1
        slot = (int(diff[0]), int(np.nonzero(t)[0][0]))
        assert owner.setdefault(slot, (row, col)) == (row, col)


def test_rejects_non_trits_and_bad_bytes():
    with pytest.raises(ValueError):
        oracle.pack_b3(np.full((1, 64), 2, np.int8))
    buf = oracle.pack_b3(np.zeros((16, 64), np.int8))
    buf[5] = 1  # no code
    with pytest.raises(ValueError):
        oracle.unpack_b3(buf, 16, 64)


@pytest.mark.parametrize("m,n,k", [(1, 33, 320), (3, 40, 704), (2, 17, 2560)])
def test_forward_b3_equals_forward_2bit(m, n, k):
    """The whole layer read from the base-3 buffer equals the pinned 2-bit
    forward of the same trits (same gamma, activations, outputs)."""
    rng = np.random.default_rng(m * 100 + n + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    g = oracle.absmean(w)
    q = oracle.ternarize(w, g)
    x = datagen.activations_bf16(int(rng.integers(1 << 40)), m, k, rng.choice(k, 4, replace=False), 20.0)
    got = oracle.bitlinear_forward_b3(oracle.pack_b3(q), g, x, n)
    want = oracle.bitlinear_forward(oracle.pack(q), g, x, n)
    for a, b in zip(got, want):
        np.testing.assert_array_equal(a, b)


def test_ternarize_pack_b3_on_a_workload_matrix():
    w = datagen.weights(datagen.stream_id(datagen.WORKLOAD_STACK_2B, 0, 1, datagen.TENSOR_W), 256, 2560)
    buf, g = oracle.ternarize_pack_b3(w)
    assert g == oracle.absmean(w)
    np.testing.assert_array_equal(oracle.unpack_b3(buf, 256, 2560), oracle.ternarize(w, g))
