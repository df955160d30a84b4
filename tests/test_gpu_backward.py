"""GPU parity of the straight-through backward against the CPU oracle.

Bar: the transposed packing bit-exact; dx within the fp32 accumulation bound
of the oracle's exactly rounded value: |dx - want| <= (n + 2) * 2^-24 * gamma *
sum_j |dy[i][j]| + one fp32 ulp of want (the products dy * q are exact; only
the order of the fp32 sums differs).  Shapes span several 128-row x 64-token
workgroups, ragged token counts, a partial last 256-column step, and the
2B-shaped layers at full size (sampled token rows).
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import ternary_weight_absmean_amd as bl
from _gpu import bf16, f32, host, say, u8

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected only where a GPU exists
    pytest.skip("no GPU visible", allow_module_level=True)


def dy_bits(rng, m, n):
    return datagen.f32_to_bf16((rng.standard_normal((m, n)) * 0.01).astype(np.float32))


def assert_dx_close(got, want, dy, gamma, n):
    dyf = datagen.bf16_to_f32(dy).reshape(dy.shape).astype(np.float64)
    bound = (n + 2) * 2.0 ** -24 * float(gamma) * np.abs(dyf).sum(axis=1, keepdims=True)
    bound = bound + np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} differ beyond the bound; worst {np.max(err - bound):.3e}"


@pytest.mark.parametrize("n,k", [(64, 64), (128, 192), (320, 640), (2560, 6912), (13824, 2560)])
def test_pack_transposed_matches_oracle(n, k):
    rng = np.random.default_rng(n + k)
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    packed = oracle.pack(q)
    say(f"bl_pack_transposed n={n} k={k}")
    got = host(bl.bl_pack_transposed(u8(packed), n, k))
    want = oracle.pack_transposed(packed, n, k)
    mism = np.nonzero(got != want)[0]
    assert mism.size == 0, f"{mism.size} bytes differ, first at {mism[:5]}"


@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (5, 128, 320), (64, 256, 256), (70, 320, 192), (130, 1024, 640),
                                   (17, 2560, 2560), (3, 6912, 128)])
def test_backward_x_matches_oracle(m, n, k):
    rng = np.random.default_rng(m * 7 + n + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    packed, gamma = oracle.ternarize_pack(w)
    dy = dy_bits(rng, m, n)
    dy[0, :3] = 0
    say(f"bl_bitlinear_backward_x m={m} n={n} k={k}")
    packed_d, gamma_d = bl.bl_ternarize_pack(f32(w))
    packed_t = bl.bl_pack_transposed(packed_d, n, k)
    dx = host(bl.bl_bitlinear_backward_x(packed_t, gamma_d, bf16(dy), k))
    want = oracle.backward_x(packed, gamma, dy, n, k)
    assert_dx_close(dx, want, dy, gamma, n)


@pytest.mark.parametrize("name,n,k", [("gate_up", 13824, 2560), ("down", 2560, 6912)])
def test_backward_x_2b_layer_sampled(name, n, k):
    """2B-shaped layer at full size, 2048 tokens; the oracle checks sampled tokens."""
    rng = np.random.default_rng(n)
    m = 2048
    w = datagen.weights(int(rng.integers(1 << 40)), n, k)
    packed, gamma = oracle.ternarize_pack(w)
    dy = dy_bits(rng, m, n)
    say(f"bl_bitlinear_backward_x 2B {name} m={m}")
    packed_t = bl.bl_pack_transposed(u8(packed), n, k)
    dx = host(bl.bl_bitlinear_backward_x(packed_t, torch.tensor([gamma], device="cuda"), bf16(dy), k))
    toks = np.unique(np.concatenate([[0, m - 1], rng.choice(m, size=6, replace=False)]))
    want = oracle.backward_x(packed, gamma, dy[toks], n, k)
    assert_dx_close(dx[toks], want, dy[toks], gamma, n)


def test_backward_x_zero_gamma_and_empty():
    rng = np.random.default_rng(1)
    n, k, m = 128, 128, 3
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    packed_t = bl.bl_pack_transposed(u8(oracle.pack(q)), n, k)
    dx = host(bl.bl_bitlinear_backward_x(packed_t, torch.zeros(1, device="cuda"), bf16(dy_bits(rng, m, n)), k))
    assert not dx.any()
    empty = bl.bl_bitlinear_backward_x(packed_t, torch.ones(1, device="cuda"),
                                       torch.zeros((0, n), dtype=torch.bfloat16, device="cuda"), k)
    assert empty.shape == (0, k)


def assert_dw_close(got, want, dy, xq, alpha):
    m = dy.shape[0]
    dyf = datagen.bf16_to_f32(dy).reshape(dy.shape).astype(np.float64)
    mag = (np.abs(dyf) * alpha.astype(np.float64)[:, None]).T @ np.abs(xq.astype(np.float64)) / 127
    bound = (m + 2) * 2.0 ** -24 * mag + 2 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} differ beyond the bound; worst {np.max(err - bound):.3e}"


def w_case(rng, m, n, k):
    dy = dy_bits(rng, m, n)
    x = datagen.activations_bf16(int(rng.integers(1 << 40)), m, k, rng.choice(k, size=min(8, k), replace=False), 20.0)
    xq, alpha = oracle.quant_act(x)
    return dy, xq, alpha


@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (5, 128, 320), (64, 256, 256), (70, 320, 192), (130, 1024, 640),
                                   (200, 64, 2560)])
def test_backward_w_matches_oracle(m, n, k):
    rng = np.random.default_rng(m * 11 + n + 3 * k)
    dy, xq, alpha = w_case(rng, m, n, k)
    say(f"bl_bitlinear_backward_w m={m} n={n} k={k}")
    dw = host(bl.bl_bitlinear_backward_w(bf16(dy), torch.from_numpy(xq).cuda(), torch.from_numpy(alpha).cuda()))
    want = oracle.backward_w(dy, xq, alpha)
    assert_dw_close(dw, want, dy, xq, alpha)


@pytest.mark.parametrize("name,n,k", [("gate_up", 13824, 2560), ("down", 2560, 6912)])
def test_backward_w_2b_layer_sampled(name, n, k):
    """2B-shaped layer, 2048 tokens; the oracle checks sampled rows of dw."""
    rng = np.random.default_rng(n + 1)
    m = 2048
    dy, xq, alpha = w_case(rng, m, n, k)
    say(f"bl_bitlinear_backward_w 2B {name} m={m}")
    dw = host(bl.bl_bitlinear_backward_w(bf16(dy), torch.from_numpy(xq).cuda(), torch.from_numpy(alpha).cuda()))
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=6, replace=False)]))
    want = oracle.backward_w(np.ascontiguousarray(dy[:, rows]), xq, alpha)
    assert_dw_close(dw[rows], want, np.ascontiguousarray(dy[:, rows]), xq, alpha)


def test_backward_w_empty_tokens_gives_zero():
    dw = bl.bl_bitlinear_backward_w(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"),
                                    torch.zeros((0, 128), dtype=torch.int8, device="cuda"),
                                    torch.zeros(0, dtype=torch.float32, device="cuda"),
                                    dw=torch.full((64, 128), 7.0, device="cuda"))
    assert not host(dw).any()
