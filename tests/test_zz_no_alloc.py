"""The allocation-free packer against the workspace packer, through the C ABI.

bl_ternarize_pack_noalloc keeps its exponent bins in the library's static
device array instead of a caller workspace; for callers that cannot allocate
(graph capture, serving loops) it must give exactly bl_ternarize_pack's gamma
and packed bytes.  Two calls in a row, the second on a smaller matrix, check
that what the first left in the shared array does not leak into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

import datagen
import ternary_weight_absmean_amd as bl
from _gpu import DEV, f32, host, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected only where a GPU exists
    pytest.skip("no GPU visible", allow_module_level=True)

lib = bl.library()
vp = ctypes.c_void_p


def pack_both(w_np):
    n, k = w_np.shape
    w = f32(w_np)
    nbytes = bl.bl_packed_bytes(n, k)
    ws = torch.empty(bl.bl_ternarize_pack_workspace_bytes(n, k), dtype=torch.uint8, device=DEV)
    p_ref = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    g_ref = torch.empty(1, dtype=torch.float32, device=DEV)
    # outputs of the allocation-free call prefilled with garbage: every byte must be written
    p_na = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=DEV)
    g_na = torch.full((1,), -7.0, dtype=torch.float32, device=DEV)
    s = vp(torch.cuda.current_stream(DEV).cuda_stream)
    say(f"bl_ternarize_pack and bl_ternarize_pack_noalloc n={n} k={k}")
    assert lib.bl_ternarize_pack(vp(w.data_ptr()), n, k, vp(p_ref.data_ptr()), vp(g_ref.data_ptr()),
                                 vp(ws.data_ptr()), ws.numel(), s) == 0
    assert lib.bl_ternarize_pack_noalloc(vp(w.data_ptr()), n, k, vp(p_na.data_ptr()), vp(g_na.data_ptr()), s) == 0
    torch.cuda.synchronize()
    assert host(g_na).view(np.uint32)[0] == host(g_ref).view(np.uint32)[0], (host(g_na), host(g_ref))
    assert torch.equal(p_na, p_ref), "packed bytes differ"
    return host(g_ref)[0]


def test_noalloc_matches_workspace_packer_twice_shrinking():
    wl = datagen.WORKLOAD_STACK_2B
    # first: the 2B gate+up matrix (13824 x 2560); second: a smaller ragged one
    # with a different gamma, so bins left from the first call would show
    name, k, n = datagen.STACK_2B_PROJ[2]
    g1 = pack_both(datagen.weights(datagen.stream_id(wl, 0, 2, datagen.TENSOR_W), n, k))
    rng = np.random.default_rng(5)
    w2 = (rng.standard_normal((33, 320)) * 0.5).astype(np.float32)
    g2 = pack_both(w2)
    assert g1 != g2


def test_noalloc_repeated_calls_are_identical():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((100, 1024)) * 0.02).astype(np.float32)
    first = pack_both(w)
    assert pack_both(w) == first
