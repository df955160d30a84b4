"""GPU parity of the five-trits-per-byte weight code against the CPU oracle.

bl_ternarize_pack_b3 must give the oracle's gamma and every packed byte bit
for bit; bl_bitlinear_b3 the oracle's int8 activations, alpha and int32
accumulators exactly and bf16 outputs within one ulp (the oracle reads each
trit from the same base-3 buffer), and exactly the outputs of the 2-bit path
on the same weights.  Shapes cover one and several super-tiles per wave, the
partial last super-tile of a row (k not a multiple of 320), ragged row bands,
one and two row bands per workgroup, four and eight waves, every activation
slot count, several tokens, and the 2B- and 70B-shaped matrices at full size.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import ternary_weight_absmean_amd as bl
from _gpu import assert_bf16_within_one_ulp, bf16, f32, host, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected only where a GPU exists
    pytest.skip("no GPU visible", allow_module_level=True)


def check_pack_b3(w):
    n, k = w.shape
    say(f"bl_ternarize_pack_b3 n={n} k={k}")
    packed, gamma = bl.bl_ternarize_pack_b3(f32(w))
    want_packed, want_gamma = oracle.ternarize_pack_b3(w)
    assert host(gamma).view(np.uint32)[0] == np.float32(want_gamma).view(np.uint32)
    got = host(packed)
    assert got.size == want_packed.size
    mism = np.nonzero(got != want_packed)[0]
    assert mism.size == 0, f"{mism.size} packed bytes differ, first at {mism[:5]}"
    return packed, gamma, want_packed, want_gamma


@pytest.mark.parametrize("n,k", [(1, 64), (16, 320), (17, 384), (40, 2560), (33, 6912), (5, 8192), (20, 704)])
def test_pack_b3_small_and_ragged(n, k):
    rng = np.random.default_rng(n * 17 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    g = oracle.absmean(w)
    d = np.float32(g + np.float32(1e-5))
    # weights on the rounding boundary d / 2 and next to it
    w.ravel()[1:5] = [d * np.float32(0.5), -d * np.float32(0.5), np.nextafter(d * np.float32(0.5), 1), d]
    check_pack_b3(w)


@pytest.mark.parametrize("proj", range(4))
def test_pack_b3_2b_layer0(proj):
    name, k, n = datagen.STACK_2B_PROJ[proj]
    check_pack_b3(datagen.weights(datagen.stream_id(datagen.WORKLOAD_STACK_2B, 0, proj, datagen.TENSOR_W), n, k))


def check_bitlinear_b3(w, x):
    n, k = w.shape
    m = x.shape[0]
    packed, gamma, want_packed, want_gamma = check_pack_b3(w)
    say(f"bl_bitlinear_b3 m={m} n={n} k={k}")
    acc, y, xq, alpha = bl.bl_bitlinear_b3(packed, gamma, bf16(x), n)
    want_y, want_acc, want_xq, want_alpha = oracle.bitlinear_forward_b3(want_packed, want_gamma, x, n)
    np.testing.assert_array_equal(host(xq), want_xq)
    np.testing.assert_array_equal(host(alpha).view(np.uint32), want_alpha.view(np.uint32))
    np.testing.assert_array_equal(host(acc), want_acc)
    assert_bf16_within_one_ulp(host(y), want_y)
    # the y-only call writes the same values
    _, y2, _, _ = bl.bl_bitlinear_b3(packed, gamma, bf16(x), n, acc=False)
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    return acc, y


@pytest.mark.parametrize("m,n,k", [
    # one band, one wave's share, partial super-tile; four waves, 2 slots
    (1, 33, 64), (1, 16, 320), (1, 40, 704), (1, 2560, 2560), (1, 48, 3840),
    # eight waves: 2, 4, 8 and 16 activation slots (13, 26, 90 and 200 super-tiles)
    (1, 40, 3904), (1, 2560, 6912), (1, 48, 8192), (1, 100, 28672), (1, 24, 64000),
    # two row bands per workgroup (>= 512 bands with short rows, >= 1024 any), ragged last band
    (1, 8200, 2560), (1, 16400, 704), (1, 17000, 8192),
    # a whole band per wave (>= 2048 bands): ragged last workgroup, partial last super-tile,
    # up to 2 quantization slots per thread (4 slots: the 70B gate+up below), two tokens
    (1, 32784, 704), (1, 40000, 2560), (1, 32768, 6912), (2, 32784, 320),
    # several tokens: one pass per token
    (2, 70, 2624), (5, 48, 6912), (16, 33, 320), (64, 40, 2560)])
def test_bitlinear_b3_matches_oracle(m, n, k):
    rng = np.random.default_rng(m * 131 + n * 7 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    cols = rng.choice(k, size=min(8, k), replace=False)
    x = datagen.activations_bf16(int(rng.integers(1 << 40)), m, k, cols, 20.0)
    if m >= 2:
        x[1] = 0  # an all-zero token
    check_bitlinear_b3(w, x)


def test_bitlinear_b3_equals_2bit_path():
    """Same weights, same token: the base-3 and 2-bit products give the same
    int32 sums and the same bf16 bits (the rescale is evaluated the same way)."""
    rng = np.random.default_rng(11)
    n, k = 3840, 2560
    w = f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = bf16(datagen.activations_bf16(123, 1, k, rng.choice(k, 8, replace=False), 20.0))
    p2, g2 = bl.bl_ternarize_pack(w)
    p3, g3 = bl.bl_ternarize_pack_b3(w)
    say("bl_bitlinear vs bl_bitlinear_b3")
    acc2, y2, _, _ = bl.bl_bitlinear(p2, g2, x, n)
    acc3, y3, _, _ = bl.bl_bitlinear_b3(p3, g3, x, n)
    torch.cuda.synchronize()
    assert torch.equal(g2, g3)
    assert torch.equal(acc2, acc3)
    assert torch.equal(y2.view(torch.int16), y3.view(torch.int16))


@pytest.mark.parametrize("proj", range(4))
def test_bitlinear_b3_2b_layer0_decode(proj):
    """The 2B-shaped layer-0 matrices at one token (benchmark inputs), every output."""
    wl = datagen.WORKLOAD_STACK_2B
    name, k, n = datagen.STACK_2B_PROJ[proj]
    w = datagen.weights(datagen.stream_id(wl, 0, proj, datagen.TENSOR_W), n, k)
    cols = datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS)
    x = datagen.activations_bf16(datagen.stream_id(wl, 0, proj, datagen.TENSOR_X), 1, k, cols,
                                 datagen.STACK_2B_OUTLIER_MULT)
    check_bitlinear_b3(w, x)


@pytest.mark.parametrize("proj", [0, 1])
def test_bitlinear_b3_70b_decode(proj):
    """The 70B-shaped gate+up (8192 -> 57344) and down (28672 -> 8192) at one
    token with the benchmark's seeded input: every output."""
    wl = datagen.WORKLOAD_70B
    name, k, n = datagen.LAYER_70B_PROJ[proj]
    w = datagen.weights(datagen.stream_id(wl, 0, proj, datagen.TENSOR_W), n, k)
    cols = datagen.outlier_columns(wl, k, datagen.n_outliers_70b(k))
    x = datagen.activations_bf16(datagen.stream_id(wl, 0, proj, datagen.TENSOR_X) + 1, 1, k, cols,
                                 datagen.LAYER_70B_OUTLIER_MULT)
    check_bitlinear_b3(w, x)


def test_bitlinear_b3_empty_is_a_noop():
    buf = torch.full((bl.bl_packed_bytes_b3(16, 320),), 128, dtype=torch.uint8, device="cuda")
    g = f32(np.array([1.0]))
    acc, y, xq, alpha = bl.bl_bitlinear_b3(buf, g, bf16(np.zeros((0, 320), np.uint16)), 16)
    assert acc.shape == (0, 16) and y.shape == (0, 16)
