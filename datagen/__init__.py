"""Seeded synthetic inputs for the BitLinear W1.58A8 layer (shared by the
oracle side and the GPU side; holds none of the layer's arithmetic).

Recipes, in the shapes of the BitNet b1.58 workloads:

* weights: fp32, ``0.02 * z`` with z ~ N(0, 1), one stream per matrix;
* activations: bf16, ``z`` per element, with a fixed set of outlier channels
  (columns) multiplied by a factor before rounding to bf16;
* outlier channels: drawn without replacement per distinct width K, shared by
  every token and every layer of that width.

The generator is a counter-based SplitMix64 with Box-Muller deviates (see
``gen.c``), so any element can be regenerated independently of the others.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libdatagen.so")

BASE_SEED = 20260101

# Stream-id plan: one id per (workload, layer, projection, tensor).
TENSOR_W = 0
TENSOR_X = 1
TENSOR_OUTLIERS = 2


def stream_id(workload: int, layer: int, proj: int, tensor: int) -> int:
    return ((workload * 1000 + layer) * 100 + proj) * 10 + tensor


def build(force: bool = False) -> str:
    """Compile ``libdatagen.so`` with gcc (OpenMP over elements)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               os.path.join(_HERE, "gen.c"), "-o", _SO + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.dg_normal_f32.argtypes = [u64, u64, ctypes.c_double, i64, p]
        lib.dg_normal_f32.restype = None
        lib.dg_normal_bf16.argtypes = [u64, u64, i64, i64, p, i64, ctypes.c_double, p]
        lib.dg_normal_bf16.restype = None
        lib.dg_pick_columns.argtypes = [u64, u64, i64, i64, p]
        lib.dg_pick_columns.restype = ctypes.c_int
        lib.dg_raw_u64.argtypes = [u64, u64, i64, p]
        lib.dg_raw_u64.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def normal_f32(stream: int, n: int, scale: float = 1.0, seed: int = BASE_SEED,
               out: np.ndarray | None = None) -> np.ndarray:
    """``n`` fp32 values ``(float)(scale * z_i)``."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == n
    _load().dg_normal_f32(seed, stream, float(scale), n, _ptr(out))
    return out


def weights(stream: int, n: int, k: int, sigma: float = 0.02, seed: int = BASE_SEED) -> np.ndarray:
    """fp32 weight matrix ``[n][k]`` (output rows x input columns), N(0, sigma^2)."""
    return normal_f32(stream, n * k, sigma, seed).reshape(n, k)


def pick_columns(stream: int, k: int, n_pick: int, seed: int = BASE_SEED) -> np.ndarray:
    out = np.empty(n_pick, dtype=np.int32)
    if n_pick:
        rc = _load().dg_pick_columns(seed, stream, k, n_pick, _ptr(out))
        if rc != 0:
            raise ValueError("n_pick must be in [0, k]")
    return out


def activations_bf16(stream: int, m: int, k: int, outlier_cols=None, outlier_mult: float = 1.0,
                     seed: int = BASE_SEED) -> np.ndarray:
    """bf16 activations ``[m][k]`` as uint16 bit patterns."""
    cols = np.zeros(0, np.int32) if outlier_cols is None else np.ascontiguousarray(outlier_cols, np.int32)
    out = np.empty((m, k), dtype=np.uint16)
    _load().dg_normal_bf16(seed, stream, m, k, _ptr(cols), cols.size, float(outlier_mult), _ptr(out))
    return out


def raw_u64(stream: int, n: int, seed: int = BASE_SEED) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().dg_raw_u64(seed, stream, n, _ptr(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 bit patterns, nearest-even (finite inputs).  Used only
    to hand-craft activation inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Workload shapes (BitNet b1.58 2B-shaped and 70B-shaped BitLinears)
# --------------------------------------------------------------------------

# 2B-shaped stack: 30 layers, hidden 2560; (name, K in, N out)
STACK_2B_LAYERS = 30
STACK_2B_PROJ = (("qkv", 2560, 3840), ("o", 2560, 2560), ("gate_up", 2560, 13824), ("down", 6912, 2560))
STACK_2B_OUTLIERS = 8          # outlier channels per width
STACK_2B_OUTLIER_MULT = 20.0

# 70B-shaped layer: hidden 8192, FFN 28672
LAYER_70B_PROJ = (("gate_up", 8192, 57344), ("down", 28672, 8192))
LAYER_70B_OUTLIER_FRAC = 0.001
LAYER_70B_OUTLIER_MULT = 30.0
LAYER_70B_LAYERS = 80

WORKLOAD_SINGLE = 1     # one 2560x2560 BitLinear, M = 1
WORKLOAD_STACK_2B = 2   # 2B-shaped stack (decode M = 1, batched decode, prefill)
WORKLOAD_70B = 5        # 70B-shaped layer


def outlier_columns(workload: int, k: int, n_pick: int) -> np.ndarray:
    """Outlier channels for one width ``k`` of a workload (same for all layers)."""
    return pick_columns(9_000_000_000 + workload * 1_000_000 + k, k, n_pick)


def n_outliers_70b(k: int) -> int:
    return int(round(LAYER_70B_OUTLIER_FRAC * k))
