"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Bar: bytes, trits, int8 activations and int32 accumulators bit-exact; gamma
and alpha bit-exact (fp32 values the method rounds once); bf16 outputs within
one bf16 ulp of the oracle's (relative <= 7.8e-3), with exact zeros kept.
Shapes span several 16x64 tiles, ragged row counts and K tails that do not
fill a 1 KiB group.  The workload cases use the BitNet b1.58 2B- and 70B-shaped
layers at full size:
  * the single 2560 x 2560 decode and every one of the 120 matrices of the
    30-layer 2B-shaped stack (each has its own gamma): packed bytes and gamma
    bit for bit, then the decode call at one token with the benchmark's seeded
    input, every output;
  * batched decode (4, 16, 64 tokens) on the 2B layer-0 shapes, every output;
  * the 2B prefill (2048 tokens) of gate+up and down, every output, through
    both bl_linear and the benchmark's bl_bitlinear;
  * the 70B-shaped layer at 1 and 16 tokens, every output; at 1024 tokens,
    every output row of 64 sampled tokens (the oracle would take minutes for
    all 1024).
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import ternary_weight_absmean_amd as bl
from _gpu import DEV, assert_bf16_within_one_ulp, bf16, f32, host, i8, say, u8

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected only where a GPU exists
    pytest.skip("no GPU visible", allow_module_level=True)


def valid_bytes():
    return np.array([a | (b << 2) | (c << 4) | (d << 6) for a in range(3) for b in range(3)
                     for c in range(3) for d in range(3)], np.uint8)


# ---------------------------------------------------------------- quantizer


def check_quant(x_bits):
    m, k = x_bits.shape
    say(f"bl_quant_act m={m} k={k}")
    xq, alpha = bl.bl_quant_act(bf16(x_bits))
    want_q, want_a = oracle.quant_act(x_bits)
    np.testing.assert_array_equal(host(xq), want_q)
    np.testing.assert_array_equal(host(alpha).view(np.uint32), want_a.view(np.uint32))


@pytest.mark.parametrize("m,k", [(1, 64), (2, 128), (3, 192), (17, 320), (100, 2560), (5, 6912), (3, 16384), (2, 12352)])
def test_quant_small_and_ragged(m, k):
    rng = np.random.default_rng(m * 7 + k)
    x = datagen.f32_to_bf16(rng.standard_normal((m, k)) * 10.0 ** rng.uniform(-4, 4, size=(m, 1)))
    check_quant(x)


def test_quant_edge_rows():
    k = 128
    rows = [np.zeros(k), np.full(k, -3.0), np.linspace(-127, 127, k), np.full(k, 1e-30)]
    tie = np.zeros(k)
    tie[:7] = [127, 2.5, -3.5, 0.5, -0.5, 1.5, -1.5]  # s = 1: ties go to even
    rows.append(tie)
    big = np.zeros(k)
    big[3] = -3.0e38
    big[4] = 1.0
    rows.append(big)
    check_quant(datagen.f32_to_bf16(np.array(rows)))


@pytest.mark.parametrize("m,k", [(1, 2560), (64, 6912), (16, 8192), (1, 28672), (2048, 2560), (1024, 28672)])
def test_quant_workload_widths(m, k):
    n_out = 8 if k in (2560, 6912) else datagen.n_outliers_70b(k)
    mult = 20.0 if k in (2560, 6912) else 30.0
    wl = datagen.WORKLOAD_STACK_2B if k in (2560, 6912) else datagen.WORKLOAD_70B
    cols = datagen.outlier_columns(wl, k, n_out)
    check_quant(datagen.activations_bf16(datagen.stream_id(wl, 0, 0, 1) + k, m, k, cols, mult))


# ---------------------------------------------------------------- weight packer


def check_pack(w):
    n, k = w.shape
    say(f"bl_ternarize_pack n={n} k={k}")
    packed, gamma = bl.bl_ternarize_pack(f32(w))
    want_packed, want_gamma = oracle.ternarize_pack(w)
    got_gamma = host(gamma)
    assert got_gamma.view(np.uint32)[0] == np.float32(want_gamma).view(np.uint32), (got_gamma[0], want_gamma)
    got = host(packed)
    assert got.size == want_packed.size
    mism = np.nonzero(got != want_packed)[0]
    assert mism.size == 0, f"{mism.size} packed bytes differ, first at {mism[:5]}"
    return packed


@pytest.mark.parametrize("n,k", [(1, 64), (5, 128), (16, 64), (17, 192), (40, 320), (33, 2560)])
def test_pack_small_and_ragged(n, k):
    rng = np.random.default_rng(n * 31 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    # weights exactly on the rounding boundaries +-0.5 * (gamma + eps) and +-1.5 * (gamma + eps)
    g = oracle.absmean(w)
    d = np.float32(g + np.float32(1e-5))
    w.ravel()[1:5] = [d * np.float32(0.5), -d * np.float32(0.5), d * np.float32(1.5), np.nextafter(d * np.float32(0.5), 1)]
    check_pack(w)


def test_pack_rounding_boundary_at_final_gamma():
    """Weights at and next to the rounding boundary d / 2 (d = gamma + 1e-5)
    of the matrix's own final gamma: the inserted values change gamma, so
    they are placed again until gamma no longer moves.  The oracle divides
    and rounds; the packed codes must agree bit for bit."""
    rng = np.random.default_rng(77)
    n, k = 64, 1024
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    pos = rng.choice(n * k, size=208, replace=False)
    near = rng.uniform(0.999, 1.001, size=200)
    signs = np.where(rng.random(200) < 0.5, -1.0, 1.0)
    g = None
    for _ in range(20):
        g = oracle.absmean(w)
        d = np.float32(np.float32(g) + np.float32(1e-5))
        h = np.float32(d * np.float32(0.5))
        up, down = np.nextafter(h, np.float32(np.inf)), np.nextafter(h, np.float32(0))
        vals = np.concatenate([[h, -h, up, -up, down, -down, d, np.float32(1.5) * d],
                               (h * near * signs).astype(np.float32)]).astype(np.float32)
        w.ravel()[pos] = vals
        if oracle.absmean(w) == g:
            break
    assert oracle.absmean(w) == g, "gamma did not settle"
    q = oracle.ternarize(w, g).ravel()[pos]
    assert (q == 0).any() and (q != 0).any()  # the inserted values straddle the boundary
    assert list(q[:6]) == [0, 0, 1, -1, 0, 0]
    check_pack(w)


def test_pack_gamma_exotic_values():
    rng = np.random.default_rng(4)
    cases = [
        np.full((16, 64), 0.02, np.float32),                                   # constant magnitude
        np.where(rng.random((16, 64)) < 0.5, -1.0, 1.0).astype(np.float32) * np.float32(3e-39),  # subnormal
        np.concatenate([np.full((1, 64), 2.0 ** 25, np.float32), np.ones((15, 64), np.float32)]),
        (rng.standard_normal((32, 128)) * 10.0 ** rng.uniform(-30, 30, size=(32, 128))).astype(np.float32),
        np.zeros((16, 64), np.float32),
    ]
    # many workgroups whose register windows differ: mostly N(0, 0.02), with
    # entries 1e6 and 1e-8 times larger and exact zeros scattered through
    w = (rng.standard_normal((600, 2560)) * 0.02).astype(np.float32)
    pick = rng.random(w.shape)
    w[pick < 0.01] *= np.float32(1e6)
    w[(pick >= 0.01) & (pick < 0.02)] *= np.float32(1e-8)
    w[(pick >= 0.02) & (pick < 0.03)] = 0.0
    cases.append(w)
    for w in cases:
        check_pack(w)


def test_unpack_helper_matches_oracle_and_all_byte_patterns():
    rng = np.random.default_rng(8)
    n, k = 37, 320
    buf = rng.choice(valid_bytes(), size=oracle.packed_bytes(n, k))
    buf[:81] = valid_bytes()
    say("bl_unpack_ternary")
    q = bl.bl_unpack_ternary(u8(buf), n, k)
    np.testing.assert_array_equal(host(q), oracle.unpack(buf, n, k))


def test_pack_workload_2b_stack_layer0():
    for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
        w = datagen.weights(datagen.stream_id(datagen.WORKLOAD_STACK_2B, 0, pi, datagen.TENSOR_W), n, k)
        check_pack(w)


def test_pack_workload_single_2560():
    check_pack(datagen.weights(datagen.stream_id(datagen.WORKLOAD_SINGLE, 0, 0, datagen.TENSOR_W), 2560, 2560))


@pytest.mark.parametrize("proj", [0, 1])
def test_pack_workload_70b_layer(proj):
    name, k, n = datagen.LAYER_70B_PROJ[proj]
    w = datagen.weights(datagen.stream_id(datagen.WORKLOAD_70B, 0, proj, datagen.TENSOR_W), n, k)
    check_pack(w)


def test_pack_is_deterministic():
    w = datagen.weights(77, 3840, 2560)
    say("bl_ternarize_pack twice")
    p1, g1 = bl.bl_ternarize_pack(f32(w))
    p2, g2 = bl.bl_ternarize_pack(f32(w))
    assert torch.equal(p1, p2) and torch.equal(g1, g2)


# ---------------------------------------------------------------- product


def check_linear(packed_dev, gamma_dev, qw, gamma_host, x_bits=None, xq_np=None, alpha_np=None, rows=None,
                 toks=None):
    """Run bl_linear on device inputs; compare acc exactly and y within 1 ulp
    with the oracle on the (optionally sampled) token rows / output columns."""
    n, k = qw.shape
    if x_bits is not None:
        xq_np, alpha_np = oracle.quant_act(x_bits)
        xq_dev, alpha_dev = bl.bl_quant_act(bf16(x_bits))
    else:
        xq_dev, alpha_dev = i8(xq_np), f32(alpha_np)
    m = xq_np.shape[0]
    say(f"bl_linear m={m} n={n} k={k}")
    acc, y = bl.bl_linear(packed_dev, gamma_dev, xq_dev, alpha_dev, n)
    acc_h, y_h = host(acc), host(y)
    toks = np.arange(m) if toks is None else toks
    rows = np.arange(n) if rows is None else rows
    want_acc = oracle.linear_mul(qw[rows], xq_np[toks])
    np.testing.assert_array_equal(acc_h[np.ix_(toks, rows)], want_acc)
    want_y = oracle.rescale(want_acc, gamma_host, alpha_np[toks])
    assert_bf16_within_one_ulp(y_h[np.ix_(toks, rows)], want_y)
    # the y-only and acc-only forms write the same values
    _, y2 = bl.bl_linear(packed_dev, gamma_dev, xq_dev, alpha_dev, n, acc=False)
    acc2, _ = bl.bl_linear(packed_dev, gamma_dev, xq_dev, alpha_dev, n, y=False)
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16)) and torch.equal(acc2, acc)
    return acc_h, y_h


def random_layer(rng, n, k):
    """Random valid packed buffer (seeded test input) and its trits per the oracle."""
    buf = rng.choice(valid_bytes(), size=oracle.packed_bytes(n, k)).astype(np.uint8)
    return buf, oracle.unpack(buf, n, k)


@pytest.mark.parametrize("m", [1, 2, 3, 5, 16, 17, 33, 64, 65, 100])
@pytest.mark.parametrize("n,k", [(1, 64), (7, 128), (31, 192), (33, 320), (48, 1024), (20, 1088), (264, 320)])
def test_linear_brute_force_shapes(m, n, k):
    rng = np.random.default_rng(1000 * m + 10 * n + k)
    buf, qw = random_layer(rng, n, k)
    xq = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    xq[0, : min(k, 8)] = [127, -128, -127, 0, 1, -1, 127, -128][: min(k, 8)]
    alpha = datagen.bf16_to_f32(datagen.f32_to_bf16(rng.uniform(0.1, 50, size=m)))
    gamma = np.float32(0.0159)
    check_linear(u8(buf), f32(np.array([gamma])), qw, gamma, xq_np=xq, alpha_np=alpha)


@pytest.mark.parametrize("m,n,k", [(16, 16400, 1024), (5, 32800, 320), (9, 16416, 2112),
                                   # 17..64 tokens in one workgroup (four token blocks) with four row
                                   # tiles, ragged last workgroup and chunk; 16-token workgroups with
                                   # one row tile, and with two once that would make 256 workgroups
                                   (64, 8200, 320), (40, 8208, 4160), (40, 1000, 4160), (33, 2000, 2560),
                                   # 17..32 tokens in one workgroup (two token blocks, two row tiles)
                                   (20, 8200, 2560), (32, 8208, 1088),
                                   # the same token counts on a matrix with many row tiles: the GEMM
                                   (20, 32784, 128),
                                   # 2..16 tokens on rows of 8192 and more: the LDS ring with 1, 2 and 4
                                   # row tiles per workgroup, ragged last workgroup, partial last chunk
                                   (3, 40, 8256), (16, 8208, 9216), (5, 32784, 8256), (16, 33, 16448),
                                   # 17..64 tokens: 16-token workgroups (LDS-staged, and the ring with a
                                   # ragged last token block), 64-token workgroups from 512 row tiles
                                   (24, 600, 2560), (40, 100, 8256), (33, 8208, 640)])
def test_linear_multi_tile_workgroups(m, n, k):
    """Token blocks whose activation loads serve 2 or 4 row tiles per
    workgroup, with a ragged last workgroup."""
    rng = np.random.default_rng(7 * m + n + k)
    buf, qw = random_layer(rng, n, k)
    xq = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    alpha = datagen.bf16_to_f32(datagen.f32_to_bf16(rng.uniform(0.1, 50, size=m)))
    gamma = np.float32(0.0271)
    say(f"bl_linear multi-tile m={m} n={n} k={k}")
    check_linear(u8(buf), f32(np.array([gamma])), qw, gamma, xq_np=xq, alpha_np=alpha)


def test_linear_extremes():
    k, n, m = 6912, 48, 4
    qw = np.ones((n, k), np.int8)
    qw[16:32] = -1
    qw[32:, ::3] = 0
    xq = np.full((m, k), 127, np.int8)
    xq[1] = -128
    xq[2] = 0
    xq[3, ::2] = -127
    packed = oracle.pack(qw)
    alpha = np.array([127.0, 128.0, 0.0, 99.0], np.float32)
    gamma = np.float32(0.03)
    acc, y = check_linear(u8(packed), f32(np.array([gamma])), qw, gamma, xq_np=xq, alpha_np=alpha)
    assert acc[0, 0] == 127 * k and acc[1, 20] == 128 * k and (acc[2] == 0).all()


def test_linear_large_k_accumulator_range():
    k, n, m = 1 << 20, 16, 2
    qw = np.ones((n, k), np.int8)
    qw[8:] = -1
    xq = np.full((m, k), 127, np.int8)
    xq[1] = -128
    gamma = np.float32(1e-3)
    alpha = np.array([1.0, 2.0], np.float32)
    acc, _ = check_linear(u8(oracle.pack(qw)), f32(np.array([gamma])), qw, gamma, xq_np=xq, alpha_np=alpha)
    assert acc[1, 0] == -128 * k and acc[1, 15] == 128 * k


def test_linear_empty_is_a_noop():
    buf = u8(np.full(oracle.packed_bytes(16, 64), 0x55, np.uint8))
    g = f32(np.array([1.0]))
    acc, y = bl.bl_linear(buf, g, i8(np.zeros((0, 64))), f32(np.zeros(0)), 16)
    assert acc.shape == (0, 16) and y.shape == (0, 16)
    acc = torch.full((2, 0), 7, dtype=torch.int32, device=DEV)
    bl.bl_linear(buf, g, i8(np.zeros((2, 64))), f32(np.zeros(2)), 0, acc=acc, y=False)


def workload_case(workload, proj, k, n, m, outliers, mult, layer=0, sample=None):
    """Pack seeded weights on the GPU (gamma and bytes checked against the
    oracle), quantize seeded activations on the GPU, and compare the product.
    sample: (tokens, rows) to compare, either None for all of them."""
    w = datagen.weights(datagen.stream_id(workload, layer, proj, datagen.TENSOR_W), n, k)
    packed_dev = check_pack(w)
    gamma = oracle.absmean(w)
    qw = oracle.ternarize(w, gamma)
    del w
    cols = datagen.outlier_columns(workload, k, outliers)
    x = datagen.activations_bf16(datagen.stream_id(workload, layer, proj, datagen.TENSOR_X) + 7 * m, m, k, cols, mult)
    rows = toks = None
    if sample is not None:
        rng = np.random.default_rng(m + n)
        if sample[0] is not None:
            toks = np.sort(rng.choice(m, size=min(m, sample[0]), replace=False))
        if sample[1] is not None:
            rows = np.sort(rng.choice(n, size=min(n, sample[1]), replace=False))
    gamma_dev = f32(np.array([gamma]))
    check_linear(packed_dev, gamma_dev, qw, gamma, x_bits=x, rows=rows, toks=toks)


def test_linear_workload_single_2560_decode():
    workload_case(datagen.WORKLOAD_SINGLE, 0, 2560, 2560, 1, 0, 1.0)


@pytest.mark.parametrize("m", [1, 4, 16, 64])
def test_linear_workload_2b_stack_layer0(m):
    for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
        workload_case(datagen.WORKLOAD_STACK_2B, pi, k, n, m, datagen.STACK_2B_OUTLIERS if m == 1 else 0,
                      datagen.STACK_2B_OUTLIER_MULT)


def test_linear_workload_2b_stack_last_layer_decode():
    for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
        workload_case(datagen.WORKLOAD_STACK_2B, pi, k, n, 1, datagen.STACK_2B_OUTLIERS,
                      datagen.STACK_2B_OUTLIER_MULT, layer=datagen.STACK_2B_LAYERS - 1)


@pytest.mark.parametrize("proj", [2, 3])
def test_linear_workload_2b_prefill_2048(proj):
    """The 2B prefill shapes (gate+up 2560 -> 13824, down 6912 -> 2560) at
    2048 tokens: every output of the GEMM."""
    name, k, n = datagen.STACK_2B_PROJ[proj]
    workload_case(datagen.WORKLOAD_STACK_2B, proj, k, n, 2048, datagen.STACK_2B_OUTLIERS,
                  datagen.STACK_2B_OUTLIER_MULT)


@pytest.mark.parametrize("proj", [0, 1])
@pytest.mark.parametrize("m", [1, 16, 1024])
def test_linear_workload_70b(proj, m):
    """The 70B-shaped layer: every output at 1 and 16 tokens; at 1024 tokens
    every output row of 64 sampled tokens."""
    name, k, n = datagen.LAYER_70B_PROJ[proj]
    sample = (64, None) if m == 1024 else None
    workload_case(datagen.WORKLOAD_70B, proj, k, n, m, datagen.n_outliers_70b(k), datagen.LAYER_70B_OUTLIER_MULT,
                  sample=sample)


def test_linear_is_deterministic():
    rng = np.random.default_rng(3)
    buf, qw = random_layer(rng, 3840, 2560)
    xq = i8(rng.integers(-127, 128, size=(5, 2560)))
    a = f32(np.ones(5))
    g = f32(np.array([0.01]))
    say("bl_linear twice")
    acc1, y1 = bl.bl_linear(u8(buf), g, xq, a, 3840)
    acc2, y2 = bl.bl_linear(u8(buf), g, xq, a, 3840)
    assert torch.equal(acc1, acc2) and torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ---------------------------------------------------------------- whole layer in one call


@pytest.mark.parametrize("m,n,k", [
    # single-token kernel: both slot counts and eight waves (rows up to 28672), one and two row
    # tiles per workgroup (1025 row tiles), ragged last workgroup, partial last column group
    (1, 33, 64), (1, 2560, 2560), (1, 2560, 6912), (1, 100, 28672), (1, 8200, 320), (1, 16400, 2560),
    (1, 16400, 6912), (1, 17000, 7168), (1, 40, 192), (1, 1000, 2624), (1, 9000, 4160), (1, 8200, 28672),
    (1, 16400, 8192), (1, 530, 16384), (1, 16400, 10304),
    # block-quantizing kernel (rows the others do not hold): one token past 28672 columns, whose
    # activations are read twice instead of held in registers; 2-3 tokens past 8192 columns
    (1, 40, 32832), (3, 48, 10240), (2, 70, 12352),
    # 3 tokens of 8192 columns on a matrix where both fused kernels would repeat too much
    # quantization: quantizer + LDS-ring product
    (3, 43712, 8192),
    # token-block kernel: eight waves (up to 8 tokens) and sixteen, one and four row tiles (512+),
    # every chunk count per lane up to 16, ragged last workgroup and column group, m * k at its limit
    (2, 17, 320), (3, 8200, 2560), (2, 8200, 2560), (16, 16400, 1024), (5, 48, 5120), (8, 16400, 2560),
    (16, 32800, 320), (5, 2000, 6912), (4, 600, 6912), (3, 9000, 8000), (2, 70, 2624), (4, 1000, 4096),
    (4, 8000, 2560), (4, 8200, 2560), (7, 530, 2112), (6, 16400, 320), (3, 48, 2560), (4, 3840, 2560),
    (5, 40, 6912), (16, 64, 1024), (16, 31, 2560), (6, 240, 2560), (8, 160, 2560), (10, 240, 2560),
    (6, 1040, 2560), (2, 8200, 8192), (9, 100, 7232), (16, 8200, 4096), (16, 40, 4096), (12, 530, 5440),
    (5, 33, 64), (3, 20, 1088),
    # past its limits: quantizer + LDS-staged product (m * k > 65536, or more than 16 tokens) and
    # quantizer + LDS-ring product (rows of 8192 and more)
    (16, 200, 4160), (17, 40, 2560), (64, 100, 2560), (4, 33, 10240), (7, 70, 16448), (16, 40, 32768),
    (4, 16, 28672)])
def test_bitlinear_matches_oracle(m, n, k):
    """bl_bitlinear (fused quantize + product where it fits, two kernels
    otherwise) against the oracle's quantizer, product and rescale."""
    rng = np.random.default_rng(m * 131 + n * 7 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    cols = rng.choice(k, size=min(8, k), replace=False)
    x = datagen.activations_bf16(int(rng.integers(1 << 40)), m, k, cols, 20.0)
    if m >= 2:
        x[1] = 0  # an all-zero token
    say(f"bl_bitlinear m={m} n={n} k={k}")
    packed, gamma = bl.bl_ternarize_pack(f32(w))
    acc, y, xq, alpha = bl.bl_bitlinear(packed, gamma, bf16(x), n)
    want_packed, want_gamma = oracle.ternarize_pack(w)
    want_y, want_acc, want_xq, want_alpha = oracle.bitlinear_forward(want_packed, want_gamma, x, n)
    np.testing.assert_array_equal(host(xq), want_xq)
    np.testing.assert_array_equal(host(alpha).view(np.uint32), want_alpha.view(np.uint32))
    np.testing.assert_array_equal(host(acc), want_acc)
    assert_bf16_within_one_ulp(host(y), want_y)
    # y-only call writes the same bf16 values
    _, y2, _, _ = bl.bl_bitlinear(packed, gamma, bf16(x), n, acc=False)
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("layer", range(datagen.STACK_2B_LAYERS))
def test_bitlinear_2b_stack_every_matrix(layer):
    """The benchmark's own step, on every matrix of the 30-layer 2B-shaped
    stack (each has its own gamma): the packer's gamma and bytes bit for bit,
    then bl_bitlinear at one token on the benchmark's seeded input (int8
    activations, alpha and int32 exact; bf16 within one ulp), every output."""
    wl = datagen.WORKLOAD_STACK_2B
    for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
        w = datagen.weights(datagen.stream_id(wl, layer, pi, datagen.TENSOR_W), n, k)
        cols = datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS)
        x = datagen.activations_bf16(datagen.stream_id(wl, layer, pi, datagen.TENSOR_X), 1, k, cols,
                                     datagen.STACK_2B_OUTLIER_MULT)
        say(f"bl_ternarize_pack + bl_bitlinear 2B layer {layer} {name}")
        packed = check_pack(w)
        want_packed, want_gamma = oracle.ternarize_pack(w)
        del w
        gamma = f32(np.array([want_gamma]))
        acc, y, xq, alpha = bl.bl_bitlinear(packed, gamma, bf16(x), n)
        want_y, want_acc, want_xq, want_alpha = oracle.bitlinear_forward(want_packed, want_gamma, x, n)
        np.testing.assert_array_equal(host(xq), want_xq)
        np.testing.assert_array_equal(host(alpha).view(np.uint32), want_alpha.view(np.uint32))
        np.testing.assert_array_equal(host(acc), want_acc)
        assert_bf16_within_one_ulp(host(y), want_y)


@pytest.mark.parametrize("proj", [2, 3])
def test_bitlinear_2b_prefill_full(proj):
    """The benchmark's prefill call (bl_bitlinear: quantizer + GEMM) on the 2B
    layer-0 gate+up and down at 2048 tokens, with the benchmark's seeded
    input: every output."""
    wl = datagen.WORKLOAD_STACK_2B
    name, k, n = datagen.STACK_2B_PROJ[proj]
    m = 2048
    w = datagen.weights(datagen.stream_id(wl, 0, proj, datagen.TENSOR_W), n, k)
    cols = datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS)
    x = datagen.activations_bf16(datagen.stream_id(wl, 0, proj, datagen.TENSOR_X) + m, m, k, cols,
                                 datagen.STACK_2B_OUTLIER_MULT)
    say(f"bl_bitlinear 2B prefill {name} m={m}")
    check_bitlinear_sampled(w, x)


def check_bitlinear_sampled(w, x, rows=None):
    """bl_bitlinear (the benchmark's call) against the oracle's quantizer and
    product on the given output rows (all when None), every token."""
    n, k = w.shape
    packed, gamma = bl.bl_ternarize_pack(f32(w))
    acc, y, xq, alpha = bl.bl_bitlinear(packed, gamma, bf16(x), n)
    want_gamma = oracle.absmean(w)
    assert host(gamma).view(np.uint32)[0] == np.float32(want_gamma).view(np.uint32)
    qw = oracle.ternarize(w, want_gamma)
    want_xq, want_alpha = oracle.quant_act(x)
    np.testing.assert_array_equal(host(xq), want_xq)
    np.testing.assert_array_equal(host(alpha).view(np.uint32), want_alpha.view(np.uint32))
    rows = np.arange(n) if rows is None else rows
    want_acc = oracle.linear_mul(qw[rows], want_xq)
    np.testing.assert_array_equal(host(acc)[:, rows], want_acc)
    assert_bf16_within_one_ulp(host(y)[:, rows], oracle.rescale(want_acc, want_gamma, want_alpha))


@pytest.mark.parametrize("m", [4, 16, 64])
def test_bitlinear_2b_stack_batched_decode(m):
    """The benchmark's batched-decode call on the 2B layer-0 shapes: seeded
    weights, independent N(0, 1) token rows."""
    wl = datagen.WORKLOAD_STACK_2B
    for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
        w = datagen.weights(datagen.stream_id(wl, 0, pi, datagen.TENSOR_W), n, k)
        x = datagen.activations_bf16(datagen.stream_id(wl, 0, pi, datagen.TENSOR_X) + 7 * m, m, k, [], 1.0)
        say(f"bl_bitlinear 2B layer 0 {name} m={m}")
        check_bitlinear_sampled(w, x)


@pytest.mark.parametrize("proj", [0, 1])
@pytest.mark.parametrize("m", [1, 16])
def test_bitlinear_70b_decode(proj, m):
    """The benchmark's 70B-shaped decode call (full shapes, every output)."""
    wl = datagen.WORKLOAD_70B
    name, k, n = datagen.LAYER_70B_PROJ[proj]
    w = datagen.weights(datagen.stream_id(wl, 0, proj, datagen.TENSOR_W), n, k)
    cols = datagen.outlier_columns(wl, k, datagen.n_outliers_70b(k))
    x = datagen.activations_bf16(datagen.stream_id(wl, 0, proj, datagen.TENSOR_X) + m, m, k, cols,
                                 datagen.LAYER_70B_OUTLIER_MULT)
    say(f"bl_bitlinear 70B {name} m={m}")
    check_bitlinear_sampled(w, x)
