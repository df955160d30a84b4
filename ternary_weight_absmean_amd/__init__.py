"""BitLinear W1.58A8 on MI355X (gfx950): thin Python binding of ``libbitlinear.so``.

The layer is the BitNet b1.58 BitLinear (bako.co, "The BitLinear Layer and
AbsMean Quantization"; deepmox.com chapter 8, "A low-bit model is a whole-stack
design"): absmean-ternarized weights packed at 2 bits, per-token absmax int8
activations, int32 accumulation and a bf16 rescale.  Every step runs in the HIP
kernels behind the C ABI (``include/bitlinear.h``); this module only marshals
torch tensors (device memory, the current stream) into those calls.  There is
no fallback: if the library is missing, importing raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

from ._build import LIB_PATH, INCLUDE

__all__ = [
    "BitLinearError", "bl_packed_bytes", "bl_ternarize_pack_workspace_bytes", "bl_ternarize_pack",
    "bl_quant_act", "bl_linear", "bl_bitlinear", "bl_unpack_ternary", "bl_status_string", "library", "declared_symbols",
    "bl_ternarize_pack_glu", "bl_linear_glu", "bl_bitlinear_glu", "bl_pack_transposed", "bl_bitlinear_backward_x",
    "bl_backward_w_workspace_bytes", "bl_bitlinear_backward_w", "bl_ternarize_pack_noalloc",
    "bl_packed_bytes_b3", "bl_ternarize_pack_b3", "bl_bitlinear_b3",
]


class BitLinearError(RuntimeError):
    """A ``bl_*`` call returned a status other than BL_OK."""

    def __init__(self, func: str, status: int):
        super().__init__(f"{func}: {bl_status_string(status)} ({status})")
        self.status = status


# BITLINEAR_LIB may name another build of the same library (the test suite
# loads a host-sanitizer build this way); by default the in-tree build.
_LIB_FILE = os.environ.get("BITLINEAR_LIB") or LIB_PATH
if not os.path.exists(_LIB_FILE):
    raise ImportError(f"libbitlinear.so is not built ({_LIB_FILE}); run __graft_entry__.build()")

_lib = ctypes.CDLL(_LIB_FILE)
_P, _I64, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
_lib.bl_packed_bytes.argtypes = [_I64, _I64]
_lib.bl_packed_bytes.restype = _SZ
_lib.bl_ternarize_pack_workspace_bytes.argtypes = [_I64, _I64]
_lib.bl_ternarize_pack_workspace_bytes.restype = _SZ
_lib.bl_ternarize_pack.argtypes = [_P, _I64, _I64, _P, _P, _P, _SZ, _P]
_lib.bl_ternarize_pack.restype = ctypes.c_int
_lib.bl_ternarize_pack_noalloc.argtypes = [_P, _I64, _I64, _P, _P, _P]
_lib.bl_ternarize_pack_noalloc.restype = ctypes.c_int
_lib.bl_packed_bytes_b3.argtypes = [_I64, _I64]
_lib.bl_packed_bytes_b3.restype = _SZ
_lib.bl_ternarize_pack_b3.argtypes = [_P, _I64, _I64, _P, _P, _P, _SZ, _P]
_lib.bl_ternarize_pack_b3.restype = ctypes.c_int
_lib.bl_bitlinear_b3.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]
_lib.bl_bitlinear_b3.restype = ctypes.c_int
_lib.bl_quant_act.argtypes = [_P, _I64, _I64, _P, _P, _P]
_lib.bl_quant_act.restype = ctypes.c_int
_lib.bl_linear.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P]
_lib.bl_linear.restype = ctypes.c_int
_lib.bl_bitlinear.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]
_lib.bl_bitlinear.restype = ctypes.c_int
_lib.bl_unpack_ternary.argtypes = [_P, _I64, _I64, _P, _P]
_lib.bl_ternarize_pack_glu.argtypes = [_P, _I64, _I64, _P, _P, _P, _SZ, _P]
_lib.bl_ternarize_pack_glu.restype = ctypes.c_int
_lib.bl_linear_glu.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
_lib.bl_linear_glu.restype = ctypes.c_int
_lib.bl_bitlinear_glu.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]
_lib.bl_bitlinear_glu.restype = ctypes.c_int
_lib.bl_pack_transposed.argtypes = [_P, _I64, _I64, _P, _P]
_lib.bl_pack_transposed.restype = ctypes.c_int
_lib.bl_bitlinear_backward_x.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _P]
_lib.bl_bitlinear_backward_x.restype = ctypes.c_int
_lib.bl_backward_w_workspace_bytes.argtypes = [_I64, _I64, _I64]
_lib.bl_backward_w_workspace_bytes.restype = _SZ
_lib.bl_bitlinear_backward_w.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]
_lib.bl_bitlinear_backward_w.restype = ctypes.c_int
_lib.bl_unpack_ternary.restype = ctypes.c_int
_lib.bl_status_string.argtypes = [ctypes.c_int]
_lib.bl_status_string.restype = ctypes.c_char_p


def library() -> ctypes.CDLL:
    """The loaded C-ABI library (for callers that marshal pointers themselves)."""
    return _lib


def declared_symbols() -> list[str]:
    """Names of the functions declared in ``include/bitlinear.h``."""
    with open(os.path.join(INCLUDE, "bitlinear.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bl_\w+)\s*\(", text)))


def bl_status_string(status: int) -> str:
    return _lib.bl_status_string(int(status)).decode()


def _check(func: str, status: int) -> None:
    if status != 0:
        raise BitLinearError(func, status)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple | None = None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def bl_packed_bytes(n: int, k: int) -> int:
    return int(_lib.bl_packed_bytes(n, k))


def bl_ternarize_pack_workspace_bytes(n: int, k: int) -> int:
    return int(_lib.bl_ternarize_pack_workspace_bytes(n, k))


def bl_ternarize_pack(w: torch.Tensor, packed: torch.Tensor | None = None, gamma: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None):
    """fp32 weights ``[n][k]`` -> (packed uint8 [bl_packed_bytes], gamma fp32 [1])."""
    _need(w, "w", torch.float32)
    n, k = w.shape
    nbytes = bl_packed_bytes(n, k)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = bl_ternarize_pack_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=w.device)
    _check("bl_ternarize_pack", _lib.bl_ternarize_pack(_ptr(w), n, k, _ptr(packed), _ptr(gamma), _ptr(workspace),
                                                       workspace.numel(), _stream(w.device)))
    return packed, gamma


def bl_ternarize_pack_noalloc(w: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor):
    """bl_ternarize_pack into caller-provided outputs, with the library's static
    device bins instead of a workspace (the call itself allocates nothing)."""
    _need(w, "w", torch.float32)
    n, k = w.shape
    _need(packed, "packed", torch.uint8)
    _need(gamma, "gamma", torch.float32)
    if packed.numel() < bl_packed_bytes(n, k) or gamma.numel() < 1:
        raise ValueError("packed or gamma buffer too small")
    _check("bl_ternarize_pack_noalloc", _lib.bl_ternarize_pack_noalloc(_ptr(w), n, k, _ptr(packed), _ptr(gamma),
                                                                       _stream(w.device)))
    return packed, gamma


def bl_packed_bytes_b3(n: int, k: int) -> int:
    return int(_lib.bl_packed_bytes_b3(n, k))


def bl_ternarize_pack_b3(w: torch.Tensor, packed: torch.Tensor | None = None, gamma: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None):
    """fp32 weights ``[n][k]`` -> (five-trits-per-byte uint8 [bl_packed_bytes_b3], gamma fp32 [1])."""
    _need(w, "w", torch.float32)
    n, k = w.shape
    if packed is None:
        packed = torch.empty(max(bl_packed_bytes_b3(n, k), 1), dtype=torch.uint8, device=w.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=w.device)
    if workspace is None:
        workspace = torch.empty(max(bl_ternarize_pack_workspace_bytes(n, k), 16), dtype=torch.uint8, device=w.device)
    _check("bl_ternarize_pack_b3", _lib.bl_ternarize_pack_b3(_ptr(w), n, k, _ptr(packed), _ptr(gamma),
                                                             _ptr(workspace), workspace.numel(), _stream(w.device)))
    return packed, gamma


def bl_bitlinear_b3(packed: torch.Tensor, gamma: torch.Tensor, x: torch.Tensor, n: int,
                    xq: torch.Tensor | None = None, alpha: torch.Tensor | None = None,
                    acc: torch.Tensor | None | bool = True, y: torch.Tensor | None | bool = True):
    """bf16 activations ``[m][k]`` through the layer with five-trits-per-byte
    weights: returns (acc or None, y or None, xq, alpha)."""
    _need(x, "x", torch.bfloat16)
    m, k = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    if alpha is None:
        alpha = torch.empty(m, dtype=torch.float32, device=dev)
    _need(xq, "xq", torch.int8, (m, k))
    _need(alpha, "alpha", torch.float32, (m,))
    if acc is True:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    if y is True:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    acc = acc if isinstance(acc, torch.Tensor) else None
    y = y if isinstance(y, torch.Tensor) else None
    if acc is not None:
        _need(acc, "acc", torch.int32, (m, n))
    if y is not None:
        _need(y, "y", torch.bfloat16, (m, n))
    _need(packed, "packed", torch.uint8)
    if packed.numel() < bl_packed_bytes_b3(n, k):
        raise ValueError("packed buffer is smaller than bl_packed_bytes_b3(n, k)")
    _check("bl_bitlinear_b3", _lib.bl_bitlinear_b3(_ptr(packed), _ptr(gamma), _ptr(x), m, n, k, _ptr(xq),
                                                   _ptr(alpha), _ptr(acc), _ptr(y), _stream(dev)))
    return acc, y, xq, alpha


def bl_quant_act(x: torch.Tensor, xq: torch.Tensor | None = None, alpha: torch.Tensor | None = None):
    """bf16 activations ``[m][k]`` -> (int8 [m][k], per-token absmax fp32 [m])."""
    _need(x, "x", torch.bfloat16)
    m, k = x.shape
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if alpha is None:
        alpha = torch.empty(m, dtype=torch.float32, device=x.device)
    _need(xq, "xq", torch.int8, (m, k))
    _need(alpha, "alpha", torch.float32, (m,))
    _check("bl_quant_act", _lib.bl_quant_act(_ptr(x), m, k, _ptr(xq), _ptr(alpha), _stream(x.device)))
    return xq, alpha


def bl_linear(packed: torch.Tensor, gamma: torch.Tensor, xq: torch.Tensor, alpha: torch.Tensor, n: int,
              acc: torch.Tensor | None | bool = True, y: torch.Tensor | None | bool = True):
    """Packed ternary ``[n][k]`` times int8 ``[m][k]`` -> (int32 acc [m][n] or None, bf16 y [m][n] or None).

    ``acc``/``y``: a tensor to write into, True to allocate, or False/None to skip."""
    _need(xq, "xq", torch.int8)
    m, k = xq.shape
    dev = xq.device
    if acc is True:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    if y is True:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    acc = acc if isinstance(acc, torch.Tensor) else None
    y = y if isinstance(y, torch.Tensor) else None
    if acc is not None:
        _need(acc, "acc", torch.int32, (m, n))
    if y is not None:
        _need(y, "y", torch.bfloat16, (m, n))
    _need(packed, "packed", torch.uint8)
    if packed.numel() < bl_packed_bytes(n, k):
        raise ValueError("packed buffer is smaller than bl_packed_bytes(n, k)")
    _check("bl_linear", _lib.bl_linear(_ptr(packed), _ptr(gamma), _ptr(xq), _ptr(alpha), m, n, k, _ptr(acc), _ptr(y),
                                       _stream(dev)))
    return acc, y


def bl_bitlinear(packed: torch.Tensor, gamma: torch.Tensor, x: torch.Tensor, n: int,
                 xq: torch.Tensor | None = None, alpha: torch.Tensor | None = None,
                 acc: torch.Tensor | None | bool = True, y: torch.Tensor | None | bool = True):
    """bf16 activations ``[m][k]`` through the whole layer in one call:
    returns (acc or None, y or None, xq, alpha)."""
    _need(x, "x", torch.bfloat16)
    m, k = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    if alpha is None:
        alpha = torch.empty(m, dtype=torch.float32, device=dev)
    _need(xq, "xq", torch.int8, (m, k))
    _need(alpha, "alpha", torch.float32, (m,))
    if acc is True:
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    if y is True:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    acc = acc if isinstance(acc, torch.Tensor) else None
    y = y if isinstance(y, torch.Tensor) else None
    if acc is not None:
        _need(acc, "acc", torch.int32, (m, n))
    if y is not None:
        _need(y, "y", torch.bfloat16, (m, n))
    _need(packed, "packed", torch.uint8)
    if packed.numel() < bl_packed_bytes(n, k):
        raise ValueError("packed buffer is smaller than bl_packed_bytes(n, k)")
    _check("bl_bitlinear", _lib.bl_bitlinear(_ptr(packed), _ptr(gamma), _ptr(x), m, n, k, _ptr(xq), _ptr(alpha),
                                             _ptr(acc), _ptr(y), _stream(dev)))
    return acc, y, xq, alpha


def bl_ternarize_pack_glu(w: torch.Tensor, packed: torch.Tensor | None = None, gamma: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None):
    """fp32 gate+up weights ``[2f][k]`` (gate rows first) -> (packed with
    alternating gate/up row tiles, gamma fp32 [1])."""
    _need(w, "w", torch.float32)
    n2, k = w.shape
    f = n2 // 2
    nbytes = bl_packed_bytes(n2, k)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = bl_ternarize_pack_workspace_bytes(n2, k)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=w.device)
    if n2 % 2:
        raise ValueError("a gate+up matrix has an even number of rows")
    _check("bl_ternarize_pack_glu", _lib.bl_ternarize_pack_glu(_ptr(w), f, k, _ptr(packed), _ptr(gamma),
                                                               _ptr(workspace), workspace.numel(), _stream(w.device)))
    return packed, gamma


def bl_linear_glu(packed: torch.Tensor, gamma: torch.Tensor, xq: torch.Tensor, alpha: torch.Tensor, f: int,
                  h: torch.Tensor | None = None) -> torch.Tensor:
    """Gated product from int8 activations ``[m][k]``: h bf16 [m][f]."""
    _need(xq, "xq", torch.int8)
    m, k = xq.shape
    if h is None:
        h = torch.empty((m, f), dtype=torch.bfloat16, device=xq.device)
    _need(h, "h", torch.bfloat16, (m, f))
    _need(packed, "packed", torch.uint8)
    if packed.numel() < bl_packed_bytes(2 * f, k):
        raise ValueError("packed buffer is smaller than bl_packed_bytes(2f, k)")
    _check("bl_linear_glu", _lib.bl_linear_glu(_ptr(packed), _ptr(gamma), _ptr(xq), _ptr(alpha), m, f, k, _ptr(h),
                                               _stream(xq.device)))
    return h


def bl_bitlinear_glu(packed: torch.Tensor, gamma: torch.Tensor, x: torch.Tensor, f: int,
                     xq: torch.Tensor | None = None, alpha: torch.Tensor | None = None,
                     h: torch.Tensor | None = None):
    """bf16 activations ``[m][k]`` through quantization, the gate+up product
    and squared-ReLU gating: returns (h bf16 [m][f], xq, alpha)."""
    _need(x, "x", torch.bfloat16)
    m, k = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    if alpha is None:
        alpha = torch.empty(m, dtype=torch.float32, device=dev)
    if h is None:
        h = torch.empty((m, f), dtype=torch.bfloat16, device=dev)
    _need(xq, "xq", torch.int8, (m, k))
    _need(alpha, "alpha", torch.float32, (m,))
    _need(h, "h", torch.bfloat16, (m, f))
    _need(packed, "packed", torch.uint8)
    if packed.numel() < bl_packed_bytes(2 * f, k):
        raise ValueError("packed buffer is smaller than bl_packed_bytes(2f, k)")
    _check("bl_bitlinear_glu", _lib.bl_bitlinear_glu(_ptr(packed), _ptr(gamma), _ptr(x), m, f, k, _ptr(xq),
                                                     _ptr(alpha), _ptr(h), _stream(dev)))
    return h, xq, alpha


def bl_pack_transposed(packed: torch.Tensor, n: int, k: int, packed_t: torch.Tensor | None = None) -> torch.Tensor:
    """Packed q ``[n][k]`` -> packed q^T ``[k][n]`` (n % 64 == 0)."""
    _need(packed, "packed", torch.uint8)
    if packed.numel() < bl_packed_bytes(n, k):
        raise ValueError("packed buffer is smaller than bl_packed_bytes(n, k)")
    if packed_t is None:
        packed_t = torch.empty(max(bl_packed_bytes(k, n), 1), dtype=torch.uint8, device=packed.device)
    _check("bl_pack_transposed", _lib.bl_pack_transposed(_ptr(packed), n, k, _ptr(packed_t), _stream(packed.device)))
    return packed_t


def bl_bitlinear_backward_x(packed_t: torch.Tensor, gamma: torch.Tensor, dy: torch.Tensor, k: int,
                            dx: torch.Tensor | None = None) -> torch.Tensor:
    """Straight-through input gradient: dx fp32 [m][k] = gamma * dy q, from
    packed q^T (bl_pack_transposed) and dy bf16 [m][n]."""
    _need(dy, "dy", torch.bfloat16)
    m, n = dy.shape
    if dx is None:
        dx = torch.empty((m, k), dtype=torch.float32, device=dy.device)
    _need(dx, "dx", torch.float32, (m, k))
    _need(packed_t, "packed_t", torch.uint8)
    if packed_t.numel() < bl_packed_bytes(k, n):
        raise ValueError("packed_t buffer is smaller than bl_packed_bytes(k, n)")
    _check("bl_bitlinear_backward_x", _lib.bl_bitlinear_backward_x(_ptr(packed_t), _ptr(gamma), _ptr(dy), m, n, k,
                                                                   _ptr(dx), _stream(dy.device)))
    return dx


def bl_backward_w_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(_lib.bl_backward_w_workspace_bytes(m, n, k))


def bl_bitlinear_backward_w(dy: torch.Tensor, xq: torch.Tensor, alpha: torch.Tensor, dw: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Straight-through weight gradient: dw fp32 [n][k] = dy^T (alpha / 127 xq)."""
    _need(dy, "dy", torch.bfloat16)
    _need(xq, "xq", torch.int8)
    m, n = dy.shape
    k = xq.shape[1]
    _need(alpha, "alpha", torch.float32, (m,))
    if dw is None:
        dw = torch.empty((n, k), dtype=torch.float32, device=dy.device)
    _need(dw, "dw", torch.float32, (n, k))
    ws = bl_backward_w_workspace_bytes(m, n, k)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dy.device)
    _check("bl_bitlinear_backward_w", _lib.bl_bitlinear_backward_w(_ptr(dy), _ptr(xq), _ptr(alpha), m, n, k, _ptr(dw),
                                                                   _ptr(workspace), workspace.numel(),
                                                                   _stream(dy.device)))
    return dw


def bl_unpack_ternary(packed: torch.Tensor, n: int, k: int, q: torch.Tensor | None = None) -> torch.Tensor:
    """Packed buffer -> int8 trits ``[n][k]``."""
    _need(packed, "packed", torch.uint8)
    if q is None:
        q = torch.empty((n, k), dtype=torch.int8, device=packed.device)
    _check("bl_unpack_ternary", _lib.bl_unpack_ternary(_ptr(packed), n, k, _ptr(q), _stream(packed.device)))
    return q
