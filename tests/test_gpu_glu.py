"""GPU parity of the gated feed-forward front half (gate+up BitLinear with
squared-ReLU gating) against the CPU oracle on the same seeded inputs.

Bar: packed bytes, gamma, int8 activations and alpha bit-exact; h within one
bf16 ulp of the oracle's exactly rounded value, exact zeros kept.  Cases cover
every product kernel in its gated form -- the single-token and few-token
kernels (one workgroup per gate/up tile pair), the block-quantizing kernel,
the LDS-staged and direct products, every tile shape of the GEMM -- with
ragged token counts, K tails and full 2B- and 70B-shaped matrices (sampled
token rows where the oracle would take minutes).
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import ternary_weight_absmean_amd as bl
from _gpu import assert_bf16_within_one_ulp, bf16, f32, host, i8, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected only where a GPU exists
    pytest.skip("no GPU visible", allow_module_level=True)


def glu_case(rng, f, k, m, mult=20.0):
    w = (rng.standard_normal((2 * f, k)) * 0.02).astype(np.float32)
    cols = rng.choice(k, size=min(8, k), replace=False)
    x = datagen.activations_bf16(int(rng.integers(1 << 40)), m, k, cols, mult)
    return w, x


def check_pack_glu(w):
    n2, k = w.shape
    say(f"bl_ternarize_pack_glu f={n2 // 2} k={k}")
    packed, gamma = bl.bl_ternarize_pack_glu(f32(w))
    want_packed, want_gamma = oracle.ternarize_pack_glu(w)
    assert host(gamma).view(np.uint32)[0] == np.float32(want_gamma).view(np.uint32)
    got = host(packed)
    mism = np.nonzero(got != want_packed)[0]
    assert mism.size == 0, f"{mism.size} packed bytes differ, first at {mism[:5]}"
    return packed, gamma, want_packed, want_gamma


@pytest.mark.parametrize("f,k", [(16, 64), (48, 320), (160, 2560), (6912, 2560)])
def test_pack_glu_matches_oracle(f, k):
    rng = np.random.default_rng(f * 7 + k)
    w = (rng.standard_normal((2 * f, k)) * 0.02).astype(np.float32)
    check_pack_glu(w)


@pytest.mark.parametrize("m,f,k", [
    # single-token kernel: short rows, long rows (up to the kernel's 28672), K tails
    (1, 16, 64), (1, 48, 320), (1, 160, 2560), (1, 1280, 6912), (1, 16, 28672), (1, 80, 2624),
    # token-block kernel (gate/up tile pairs, four row tiles on 512+; eight and sixteen waves)
    (2, 48, 320), (3, 160, 2560), (4, 32, 4096), (3, 4096, 2560), (5, 48, 320), (8, 160, 2560),
    (16, 48, 1024), (9, 96, 6912), (3, 48, 6912),
    # block-quantizing kernel: one token past 28672 columns, two tokens past 8192
    (1, 16, 32832), (2, 48, 12352),
    # quantizer + LDS-staged product (16- and 64-token blocks) and LDS-ring product (k >= 8192)
    (17, 160, 640), (40, 96, 640), (64, 1040, 320), (5, 48, 8256),
    # 64-token workgroups (512 row tiles of the gate+up matrix, more than 32 tokens)
    (40, 4096, 320),
    # quantizer + GEMM path: past the product's token limits, ragged token blocks
    (70, 96, 1088), (130, 272, 192),
    # one token given as int8 (bl_linear_glu): four row tiles per workgroup, ragged last
    (1, 16400, 64)])
def test_bitlinear_glu_matches_oracle(m, f, k):
    rng = np.random.default_rng(m * 131 + f * 7 + k)
    w, x = glu_case(rng, f, k, m)
    if m >= 2:
        x[1] = 0  # an all-zero token: every h is +0
    packed, gamma, want_packed, want_gamma = check_pack_glu(w)
    say(f"bl_bitlinear_glu m={m} f={f} k={k}")
    h, xq, alpha = bl.bl_bitlinear_glu(packed, gamma, bf16(x), f)
    want_h, _, want_xq, want_alpha = oracle.bitlinear_glu_forward(want_packed, want_gamma, x, f)
    np.testing.assert_array_equal(host(xq), want_xq)
    np.testing.assert_array_equal(host(alpha).view(np.uint32), want_alpha.view(np.uint32))
    assert_bf16_within_one_ulp(host(h), want_h)
    # the same product from the quantized activations
    say(f"bl_linear_glu m={m} f={f} k={k}")
    h2 = bl.bl_linear_glu(packed, gamma, xq, alpha, f)
    assert_bf16_within_one_ulp(host(h2), want_h)


def test_glu_equals_gating_of_the_plain_product():
    """bl_bitlinear_glu against the plain layer on the same weights (rows in
    gate-then-up order): the oracle gating of bl_bitlinear's exact int32
    products must give the same h."""
    rng = np.random.default_rng(11)
    f, k, m = 320, 2560, 3
    w, x = glu_case(rng, f, k, m)
    packed_glu, gamma_glu = bl.bl_ternarize_pack_glu(f32(w))
    packed, gamma = bl.bl_ternarize_pack(f32(w))
    assert host(gamma_glu).view(np.uint32)[0] == host(gamma).view(np.uint32)[0]
    say("bl_bitlinear vs bl_bitlinear_glu")
    acc, _, _, alpha = bl.bl_bitlinear(packed, gamma, bf16(x), 2 * f, y=False)
    h, _, _ = bl.bl_bitlinear_glu(packed_glu, gamma_glu, bf16(x), f)
    want = oracle.glu(host(acc), host(gamma)[0], host(alpha))
    assert_bf16_within_one_ulp(host(h), want)


@pytest.mark.parametrize("m,f,k", [
    (4096, 6912, 2560),    # 256 x 128 tiles
    (2048, 6912, 2560),    # 256 x 64 tiles, short rows (the 2B prefill gate+up)
    (1024, 4096, 8192),    # 256 x 64 tiles, long rows
    (1, 28672, 8192),      # single token, 70B-shaped gate+up
])
def test_glu_workload_shapes_sampled(m, f, k):
    """Full-size gate+up matrices; the oracle computes sampled token rows."""
    rng = np.random.default_rng(m + f + k)
    w = datagen.weights(int(rng.integers(1 << 40)), 2 * f, k)
    cols = datagen.outlier_columns(datagen.WORKLOAD_70B, k, 8)
    x = datagen.activations_bf16(int(rng.integers(1 << 40)), m, k, cols, 20.0)
    say(f"bl_bitlinear_glu sampled m={m} f={f} k={k}")
    packed, gamma = bl.bl_ternarize_pack_glu(f32(w))
    h, xq, alpha = bl.bl_bitlinear_glu(packed, gamma, bf16(x), f)
    want_gamma = oracle.absmean(w)
    assert host(gamma).view(np.uint32)[0] == np.float32(want_gamma).view(np.uint32)
    qw = oracle.ternarize(w, want_gamma)
    toks = np.unique(np.concatenate([[0, m - 1], rng.choice(m, size=min(m, 6), replace=False)]))
    want_xq, want_alpha = oracle.quant_act(x[toks])
    np.testing.assert_array_equal(host(xq)[toks], want_xq)
    np.testing.assert_array_equal(host(alpha)[toks].view(np.uint32), want_alpha.view(np.uint32))
    acc = oracle.linear_mul(qw, want_xq)
    assert_bf16_within_one_ulp(host(h)[toks], oracle.glu(acc, want_gamma, want_alpha))


def test_glu_empty_is_a_noop():
    packed = torch.zeros(bl.bl_packed_bytes(32, 64), dtype=torch.uint8, device="cuda")
    gamma = torch.ones(1, dtype=torch.float32, device="cuda")
    xq = torch.zeros((0, 64), dtype=torch.int8, device="cuda")
    alpha = torch.zeros(0, dtype=torch.float32, device="cuda")
    h = bl.bl_linear_glu(packed, gamma, xq, alpha, 16)
    assert h.shape == (0, 16)
