"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function that include/bitlinear.h
declares, and reject bad arguments on the host before anything is enqueued.
Pointers passed here are never dereferenced: every call fails validation (or
has nothing to do) before touching the device.
"""
import ctypes

import pytest
import torch

import ternary_weight_absmean_amd as bl

BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_WORKSPACE, BL_ERR_HIP = range(6)
FAKE = 0x10000  # aligned, non-null, never dereferenced
lib = bl.library()


def test_exports_every_declared_symbol():
    names = bl.declared_symbols()
    assert {"bl_ternarize_pack", "bl_quant_act", "bl_linear", "bl_unpack_ternary", "bl_packed_bytes",
            "bl_ternarize_pack_workspace_bytes", "bl_status_string"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_measurement_library_exports_and_validates():
    """libblmeasure.so (the benchmark's reference kernels) exports every
    function include/blmeasure.h declares and rejects bad arguments on the host."""
    import os
    import re
    from ternary_weight_absmean_amd._build import INCLUDE, MEASURE_LIB_PATH

    with open(os.path.join(INCLUDE, "blmeasure.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(blmeasure_\w+)\s*\(", text)))
    assert names == ["blmeasure_stream_read", "blmeasure_stream_read_sink_words"]
    m = ctypes.CDLL(MEASURE_LIB_PATH)
    for name in names:
        assert hasattr(m, name), name
    m.blmeasure_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    m.blmeasure_stream_read_sink_words.argtypes = [ctypes.c_size_t]
    m.blmeasure_stream_read_sink_words.restype = ctypes.c_size_t
    assert m.blmeasure_stream_read_sink_words(1 << 30) >= 1
    assert m.blmeasure_stream_read(None, 1 << 20, FAKE, None) == 1
    assert m.blmeasure_stream_read(FAKE, 0, FAKE, None) == 1
    assert m.blmeasure_stream_read(FAKE, 1000, FAKE, None) == 1       # not whole 32 KiB steps
    assert m.blmeasure_stream_read(FAKE + 8, 1 << 20, FAKE, None) == 1  # misaligned


def test_status_strings():
    for code in range(6):
        assert bl.bl_status_string(code).startswith("BL_")
    assert "unknown" in bl.bl_status_string(99)


def test_sizes():
    assert bl.bl_packed_bytes(2560, 2560) == 2560 * 640
    assert bl.bl_packed_bytes(17, 64) == 32 * 16
    assert bl.bl_packed_bytes(0, 64) == 0
    assert bl.bl_packed_bytes(16, 63) == 0
    assert bl.bl_packed_bytes(16, 1 << 23) == 0
    WS = 256 * 8
    assert bl.bl_ternarize_pack_workspace_bytes(57344, 8192) == WS
    assert bl.bl_ternarize_pack_workspace_bytes(16, 64) == WS
    assert bl.bl_ternarize_pack_workspace_bytes(0, 64) == 0


def test_ternarize_pack_validation():
    f = lib.bl_ternarize_pack
    WS = 256 * 8
    assert f(None, 16, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_NULL
    assert f(FAKE, 16, 64, FAKE, FAKE, None, WS, None) == BL_ERR_NULL
    assert f(FAKE, 0, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    assert f(FAKE, 16, 96, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    assert f(FAKE, 16, 0, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    assert f(FAKE, 1 << 31, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    # more than 2^35 weights (the packer's grid would pass 2^32 work-items)
    assert f(FAKE, (1 << 13) + 16, 1 << 22, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    assert f(FAKE + 4, 16, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_ALIGN
    assert f(FAKE, 16, 64, FAKE + 8, FAKE, FAKE, WS, None) == BL_ERR_ALIGN
    assert f(FAKE, 16, 64, FAKE, FAKE, FAKE, WS - 1, None) == BL_ERR_WORKSPACE


def test_ternarize_pack_noalloc_validation():
    f = lib.bl_ternarize_pack_noalloc
    assert f(None, 16, 64, FAKE, FAKE, None) == BL_ERR_NULL
    assert f(FAKE, 16, 64, None, FAKE, None) == BL_ERR_NULL
    assert f(FAKE, 0, 64, FAKE, FAKE, None) == BL_ERR_SHAPE
    assert f(FAKE, 16, 96, FAKE, FAKE, None) == BL_ERR_SHAPE
    assert f(FAKE, (1 << 13) + 16, 1 << 22, FAKE, FAKE, None) == BL_ERR_SHAPE  # past 2^35 weights
    assert f(FAKE + 4, 16, 64, FAKE, FAKE, None) == BL_ERR_ALIGN
    assert f(FAKE, 16, 64, FAKE, FAKE + 2, None) == BL_ERR_ALIGN


def test_b3_entry_points_validation():
    assert bl.bl_packed_bytes_b3(16, 320) == 1024
    assert bl.bl_packed_bytes_b3(2560, 2560) == 2560 * 512
    assert bl.bl_packed_bytes_b3(17, 64) == 32 * 64
    assert bl.bl_packed_bytes_b3(16, 100) == 0
    WS = 256 * 8
    pack = lib.bl_ternarize_pack_b3
    assert pack(None, 16, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_NULL
    assert pack(FAKE, 0, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    assert pack(FAKE, 16, 96, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    assert pack(FAKE + 4, 16, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_ALIGN
    assert pack(FAKE, 16, 64, FAKE, FAKE, FAKE, WS - 1, None) == BL_ERR_WORKSPACE
    f = lib.bl_bitlinear_b3

    def call(packed=FAKE, gamma=FAKE, x=FAKE, m=1, n=16, k=64, xq=FAKE, alpha=FAKE, acc=FAKE, y=FAKE):
        return f(packed, gamma, x, m, n, k, xq, alpha, acc, y, None)

    assert call(x=None) == BL_ERR_NULL
    assert call(acc=None, y=None) == BL_ERR_NULL
    assert call(m=65) == BL_ERR_SHAPE           # more tokens than the decode call takes
    assert call(k=64064) == BL_ERR_SHAPE        # row longer than the on-chip activations
    assert call(k=100) == BL_ERR_SHAPE
    assert call(x=FAKE + 4) == BL_ERR_ALIGN
    assert call(y=FAKE + 1) == BL_ERR_ALIGN
    assert call(m=0, x=None, xq=None) == BL_OK
    assert call(n=0) == BL_OK


def test_quant_act_validation():
    f = lib.bl_quant_act
    assert f(None, 1, 64, FAKE, FAKE, None) == BL_ERR_NULL
    assert f(None, 0, 64, None, None, None) == BL_OK  # empty: pointers may be NULL
    assert f(FAKE, -1, 64, FAKE, FAKE, None) == BL_ERR_SHAPE
    assert f(FAKE, 1, 100, FAKE, FAKE, None) == BL_ERR_SHAPE
    assert f(FAKE, (1 << 23) + 1, 64, FAKE, FAKE, None) == BL_ERR_SHAPE  # past BL_MAX_M
    assert f(FAKE + 2, 1, 64, FAKE, FAKE, None) == BL_ERR_ALIGN
    assert f(FAKE, 1, 64, FAKE, FAKE + 2, None) == BL_ERR_ALIGN
    assert f(FAKE, 0, 64, FAKE, FAKE, None) == BL_OK  # empty: nothing enqueued


def test_linear_validation():
    f = lib.bl_linear
    args = dict(packed=FAKE, gamma=FAKE, xq=FAKE, alpha=FAKE, m=1, n=16, k=64, acc=FAKE, y=FAKE, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["packed"], a["gamma"], a["xq"], a["alpha"], a["m"], a["n"], a["k"], a["acc"], a["y"], a["stream"])

    assert call(packed=None) == BL_ERR_NULL
    assert call(alpha=None) == BL_ERR_NULL
    assert call(acc=None, y=None) == BL_ERR_NULL
    assert call(k=32) == BL_ERR_SHAPE
    assert call(k=(1 << 22) + 64) == BL_ERR_SHAPE
    assert call(n=-1) == BL_ERR_SHAPE
    assert call(m=1 << 20, n=1 << 21) == BL_ERR_SHAPE  # m*n >= 2^40
    assert call(xq=FAKE + 8) == BL_ERR_ALIGN
    assert call(acc=FAKE + 2) == BL_ERR_ALIGN
    assert call(y=FAKE + 1) == BL_ERR_ALIGN
    assert call(m=0) == BL_OK
    assert call(n=0) == BL_OK
    assert call(m=0, packed=None, xq=None) == BL_OK


def test_grid_limits_are_shape_errors():
    """Shapes inside the argument limits whose launch grid would pass the
    device's 2^32 work-items are rejected on the host, before anything runs:
    2^21 tokens x 2^18 outputs (m * n = 2^39 < 2^40) needs 2^24 GEMM
    workgroups of 256 work-items."""
    m, n, k = 1 << 21, 1 << 18, 64
    assert lib.bl_linear(FAKE, FAKE, FAKE, FAKE, m, n, k, FAKE, FAKE, None) == BL_ERR_SHAPE
    assert lib.bl_bitlinear(FAKE, FAKE, FAKE, m, n, k, FAKE, FAKE, FAKE, FAKE, None) == BL_ERR_SHAPE
    assert lib.bl_linear_glu(FAKE, FAKE, FAKE, FAKE, m, n // 2, k, FAKE, None) == BL_ERR_SHAPE
    assert lib.bl_bitlinear_glu(FAKE, FAKE, FAKE, m, n // 2, k, FAKE, FAKE, FAKE, None) == BL_ERR_SHAPE
    # past the row limit (2^26)
    assert lib.bl_linear(FAKE, FAKE, FAKE, FAKE, 1, (1 << 26) + 1, k, FAKE, FAKE, None) == BL_ERR_SHAPE


def test_unpack_validation():
    f = lib.bl_unpack_ternary
    assert f(None, 16, 64, FAKE, None) == BL_ERR_NULL
    assert f(FAKE, 16, 65, FAKE, None) == BL_ERR_SHAPE
    assert f(FAKE + 1, 16, 64, FAKE, None) == BL_ERR_ALIGN
    assert f(FAKE, 0, 64, FAKE, None) == BL_OK


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only where no GPU is visible")
def test_launch_failure_maps_to_hip_error_without_a_device():
    # Valid arguments, but the HIP runtime has no device to launch on.
    assert lib.bl_quant_act(FAKE, 1, 64, FAKE, FAKE, None) == BL_ERR_HIP


def test_python_binding_rejects_host_tensors():
    with pytest.raises(ValueError):
        bl.bl_quant_act(torch.zeros((1, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        bl.bl_ternarize_pack(torch.zeros((16, 64), dtype=torch.float32))


def test_bitlinear_validation():
    f = lib.bl_bitlinear

    def call(packed=FAKE, gamma=FAKE, x=FAKE, m=1, n=16, k=64, xq=FAKE, alpha=FAKE, acc=FAKE, y=FAKE):
        return f(packed, gamma, x, m, n, k, xq, alpha, acc, y, None)

    assert call(x=None) == BL_ERR_NULL
    assert call(xq=None) == BL_ERR_NULL
    assert call(acc=None, y=None) == BL_ERR_NULL
    assert call(k=100) == BL_ERR_SHAPE
    assert call(m=-2) == BL_ERR_SHAPE
    assert call(x=FAKE + 4) == BL_ERR_ALIGN
    assert call(xq=FAKE + 1) == BL_ERR_ALIGN
    assert call(m=0, x=None, xq=None, alpha=None) == BL_OK


def test_glu_entry_points_validation():
    WS = 256 * 8
    pack = lib.bl_ternarize_pack_glu
    assert pack(None, 16, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_NULL
    assert pack(FAKE, 24, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE   # f not a multiple of 16
    assert pack(FAKE, 0, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    assert pack(FAKE, 16, 96, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE
    assert pack(FAKE, 1 << 13, 1 << 22, FAKE, FAKE, FAKE, WS, None) == BL_ERR_SHAPE  # 2f*k > 2^35
    assert pack(FAKE + 4, 16, 64, FAKE, FAKE, FAKE, WS, None) == BL_ERR_ALIGN
    assert pack(FAKE, 16, 64, FAKE, FAKE, FAKE, WS - 1, None) == BL_ERR_WORKSPACE

    lin = lib.bl_linear_glu
    assert lin(FAKE, FAKE, FAKE, FAKE, 0, 16, 64, None, None) == BL_OK     # empty
    assert lin(FAKE, FAKE, FAKE, FAKE, 1, 16, 64, None, None) == BL_ERR_NULL
    assert lin(FAKE, FAKE, FAKE, FAKE, 1, 8, 64, FAKE, None) == BL_ERR_SHAPE
    assert lin(FAKE, FAKE, FAKE, FAKE, 1, 16, 100, FAKE, None) == BL_ERR_SHAPE
    assert lin(FAKE, FAKE, FAKE + 8, FAKE, 1, 16, 64, FAKE, None) == BL_ERR_ALIGN
    assert lin(FAKE, FAKE, FAKE, FAKE, 1, 16, 64, FAKE + 1, None) == BL_ERR_ALIGN

    bit = lib.bl_bitlinear_glu
    assert bit(FAKE, FAKE, None, 0, 16, 64, None, None, None, None) == BL_OK
    assert bit(FAKE, FAKE, FAKE, 1, 16, 64, FAKE, FAKE, None, None) == BL_ERR_NULL
    assert bit(FAKE, FAKE, FAKE, 1, 17, 64, FAKE, FAKE, FAKE, None) == BL_ERR_SHAPE
    assert bit(FAKE, FAKE, FAKE, -1, 16, 64, FAKE, FAKE, FAKE, None) == BL_ERR_SHAPE
    assert bit(FAKE, FAKE, FAKE + 4, 1, 16, 64, FAKE, FAKE, FAKE, None) == BL_ERR_ALIGN


def test_backward_entry_points_validation():
    tr = lib.bl_pack_transposed
    assert tr(FAKE, 32, 64, FAKE, None) == BL_ERR_SHAPE      # n not a multiple of 64
    assert tr(FAKE, 64, 96, FAKE, None) == BL_ERR_SHAPE
    assert tr(None, 64, 64, FAKE, None) == BL_ERR_NULL
    assert tr(FAKE + 4, 64, 64, FAKE, None) == BL_ERR_ALIGN
    bx = lib.bl_bitlinear_backward_x
    assert bx(FAKE, FAKE, FAKE, 0, 64, 64, FAKE, None) == BL_OK          # empty
    assert bx(FAKE, FAKE, FAKE, 1, 96, 64, FAKE, None) == BL_ERR_SHAPE   # n % 64
    assert bx(FAKE, FAKE, FAKE, 1, (1 << 24) + 64, 64, FAKE, None) == BL_ERR_SHAPE
    assert bx(FAKE, FAKE, None, 1, 64, 64, FAKE, None) == BL_ERR_NULL
    assert bx(FAKE, FAKE, FAKE + 2, 1, 64, 64, FAKE, None) == BL_ERR_ALIGN
    assert bx(FAKE, FAKE, FAKE, 1, 64, 64, FAKE + 2, None) == BL_ERR_ALIGN


def test_backward_w_validation():
    assert bl.bl_backward_w_workspace_bytes(64, 64, 64) == 2 * (2 * 64 + 64) * 64
    assert bl.bl_backward_w_workspace_bytes(65, 128, 64) == 2 * (2 * 128 + 64) * 128
    assert bl.bl_backward_w_workspace_bytes(1, 96, 64) == 0
    bw = lib.bl_bitlinear_backward_w
    ws = bl.bl_backward_w_workspace_bytes(3, 64, 64)
    assert bw(FAKE, FAKE, FAKE, 3, 96, 64, FAKE, FAKE, ws, None) == BL_ERR_SHAPE
    assert bw(FAKE, FAKE, FAKE, 3, 64, 100, FAKE, FAKE, ws, None) == BL_ERR_SHAPE
    assert bw(FAKE, None, FAKE, 3, 64, 64, FAKE, FAKE, ws, None) == BL_ERR_NULL
    assert bw(FAKE, FAKE, FAKE, 3, 64, 64, None, FAKE, ws, None) == BL_ERR_NULL
    assert bw(FAKE + 1, FAKE, FAKE, 3, 64, 64, FAKE, FAKE, ws, None) == BL_ERR_ALIGN
    assert bw(FAKE, FAKE, FAKE, 3, 64, 64, FAKE, FAKE + 8, ws, None) == BL_ERR_ALIGN
    assert bw(FAKE, FAKE, FAKE, 3, 64, 64, FAKE, FAKE, ws - 1, None) == BL_ERR_WORKSPACE
