"""CPU oracle for the BitNet b1.58 BitLinear W1.58A8 layer.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
(``ternary_weight_absmean_amd``) never imports it, and the two share no code:
the oracle is plain serial C (``oracle.c``) behind this numpy wrapper.

Every function follows the definitions on the BitNet b1.58 pages (bako.co,
"The BitLinear Layer and AbsMean Quantization"; deepmox.com chapter 8, "A
low-bit model is a whole-stack design"); ``oracle.c`` cites each passage and
lists the readings taken where the pages are silent.

Parity status of each function (what pins it, see ``tests/test_oracle_*.py``):

* ``absmean``      -- pinned: exact rational mean (Python ``fractions``) on
  small matrices; closed forms (constant magnitudes, E|z| = sigma*sqrt(2/pi)).
* ``ternarize``    -- pinned: brute force in exact rationals for the
  round-half-even decision; threshold invariant; trit set.
* ``pack/unpack``  -- pinned: exhaustive over the 81 valid 4-trit bytes,
  round trip, code 3 rejected, per-element address formula checked by
  single-trit probes.
* ``quant_act``    -- pinned: exact rational evaluation of the fp32 steps on
  random rows; ties; range and argmax invariants; odd symmetry.
* ``linear_mul``   -- pinned: Python big-int loops and torch int64 matmul;
  equals the addition-only form.
* ``rescale``      -- pinned: exact rational product rounded to bf16 by an
  independent Python routine.
* ``b3_encode/b3_decode``, ``pack_b3/unpack_b3`` (five trits per byte) --
  pinned: all 243 five-trit patterns round-trip to 243 distinct bytes, the 13
  other bytes are rejected; hand-worked bytes; every code also decodes by the
  multiply-and-carry route; the documented digit/column property read back
  from random buffers; the 2-bit packing of the same trits unpacks equal.
* ``bitlinear_forward_b3`` -- pinned: equals ``bitlinear_forward`` on the
  2-bit packing of the same trits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
# A mutant build of oracle.c may be loaded instead (tests/test_oracle_mutants.py).
_SO_OVERRIDE = os.environ.get("BITLINEAR_ORACLE_SO")


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (IEEE fp32, no contraction)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", os.path.join(_HERE, "oracle.c"), "-o", _SO + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _SO_OVERRIDE:
            lib = ctypes.CDLL(_SO_OVERRIDE)
        else:
            if not os.path.exists(_SO):
                build()
            lib = ctypes.CDLL(_SO)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.orc_absmean.argtypes = [p, i64]
        lib.orc_absmean.restype = ctypes.c_float
        lib.orc_ternarize.argtypes = [p, i64, ctypes.c_float, p]
        lib.orc_ternarize.restype = None
        lib.orc_packed_bytes.argtypes = [i64, i64]
        lib.orc_packed_bytes.restype = i64
        lib.orc_pack.argtypes = [p, i64, i64, p]
        lib.orc_pack.restype = ctypes.c_int
        lib.orc_unpack.argtypes = [p, i64, i64, p]
        lib.orc_unpack.restype = ctypes.c_int
        lib.orc_quant_act.argtypes = [p, i64, i64, p, p]
        lib.orc_quant_act.restype = None
        lib.orc_linear_mul.argtypes = [p, p, i64, i64, i64, p]
        lib.orc_linear_mul.restype = ctypes.c_int
        lib.orc_linear_add.argtypes = [p, p, i64, i64, i64, p]
        lib.orc_linear_add.restype = ctypes.c_int
        lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
        lib.orc_bf16_from_double.restype = ctypes.c_uint16
        lib.orc_rescale.argtypes = [p, i64, i64, ctypes.c_float, p, p]
        lib.orc_rescale.restype = None
        lib.orc_bitlinear_forward.argtypes = [p, ctypes.c_float, p, i64, i64, i64, p, p, p, p]
        lib.orc_bitlinear_forward.restype = ctypes.c_int
        lib.orc_glu.argtypes = [p, i64, i64, ctypes.c_float, p, p]
        lib.orc_glu.restype = None
        lib.orc_pack_glu.argtypes = [p, i64, i64, p]
        lib.orc_pack_glu.restype = ctypes.c_int
        lib.orc_unpack_glu.argtypes = [p, i64, i64, p]
        lib.orc_unpack_glu.restype = ctypes.c_int
        lib.orc_bitlinear_glu_forward.argtypes = [p, ctypes.c_float, p, i64, i64, i64, p, p, p, p]
        lib.orc_bitlinear_glu_forward.restype = ctypes.c_int
        lib.orc_backward_x.argtypes = [p, ctypes.c_float, p, i64, i64, i64, p]
        lib.orc_backward_x.restype = ctypes.c_int
        lib.orc_backward_w.argtypes = [p, p, p, i64, i64, i64, p]
        lib.orc_backward_w.restype = None
        lib.orc_pack_transposed.argtypes = [p, i64, i64, p]
        lib.orc_pack_transposed.restype = ctypes.c_int
        lib.orc_packed_bytes_b3.argtypes = [i64, i64]
        lib.orc_packed_bytes_b3.restype = i64
        lib.orc_b3_encode.argtypes = [p]
        lib.orc_b3_encode.restype = ctypes.c_uint8
        lib.orc_b3_decode.argtypes = [ctypes.c_uint8, p]
        lib.orc_b3_decode.restype = ctypes.c_int
        lib.orc_pack_b3.argtypes = [p, i64, i64, p]
        lib.orc_pack_b3.restype = ctypes.c_int
        lib.orc_unpack_b3.argtypes = [p, i64, i64, p]
        lib.orc_unpack_b3.restype = ctypes.c_int
        lib.orc_bitlinear_forward_b3.argtypes = [p, ctypes.c_float, p, i64, i64, i64, p, p, p, p]
        lib.orc_bitlinear_forward_b3.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def absmean(w: np.ndarray) -> np.float32:
    """gamma = mean |w| over the whole matrix, exact, rounded once to fp32."""
    w = _c(w, np.float32)
    return np.float32(_load().orc_absmean(_p(w), w.size))


def ternarize(w: np.ndarray, gamma) -> np.ndarray:
    """q = clamp(round_half_even(w / (gamma + 1e-5)), -1, 1), fp32 arithmetic."""
    w = _c(w, np.float32)
    q = np.empty(w.shape, np.int8)
    _load().orc_ternarize(_p(w), w.size, float(np.float32(gamma)), _p(q))
    return q


def packed_bytes(n: int, k: int) -> int:
    return int(_load().orc_packed_bytes(n, k))


def pack(q: np.ndarray) -> np.ndarray:
    """Pack a ternary matrix ``[n][k]`` (k % 64 == 0) into the tiled 2-bit layout."""
    q = _c(q, np.int8)
    n, k = q.shape
    out = np.empty(packed_bytes(n, k), np.uint8)
    rc = _load().orc_pack(_p(q), n, k, _p(out))
    if rc != 0:
        raise ValueError(f"orc_pack failed ({rc})")
    return out


def unpack(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    if packed.size != packed_bytes(n, k):
        raise ValueError("packed buffer has the wrong size")
    q = np.empty((n, k), np.int8)
    rc = _load().orc_unpack(_p(packed), n, k, _p(q))
    if rc != 0:
        raise ValueError(f"orc_unpack failed ({rc})")
    return q


def ternarize_pack(w: np.ndarray):
    """Full weight preparation: (packed bytes, gamma)."""
    g = absmean(w)
    return pack(ternarize(w, g)), g


def quant_act(x_bf16: np.ndarray):
    """Per-token absmax int8: returns (xq [m][k] int8, alpha [m] fp32)."""
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    a = np.empty(m, np.float32)
    _load().orc_quant_act(_p(x), m, k, _p(q), _p(a))
    return q, a


def linear_mul(qw: np.ndarray, qx: np.ndarray) -> np.ndarray:
    """acc[m][n] = sum_k qx[m][k] * qw[n][k] (int32)."""
    qw = _c(qw, np.int8)
    qx = _c(qx, np.int8)
    n, k = qw.shape
    m = qx.shape[0]
    assert qx.shape[1] == k
    acc = np.empty((m, n), np.int32)
    if _load().orc_linear_mul(_p(qw), _p(qx), m, n, k, _p(acc)) != 0:
        raise OverflowError("accumulator left int32")
    return acc


def linear_add(qw: np.ndarray, qx: np.ndarray) -> np.ndarray:
    """Addition-only form of the same product."""
    qw = _c(qw, np.int8)
    qx = _c(qx, np.int8)
    n, k = qw.shape
    m = qx.shape[0]
    acc = np.empty((m, n), np.int32)
    if _load().orc_linear_add(_p(qw), _p(qx), m, n, k, _p(acc)) != 0:
        raise ValueError("weights outside {-1, 0, 1}")
    return acc


def bf16_from_double(v: float) -> int:
    return int(_load().orc_bf16_from_double(float(v)))


def rescale(acc: np.ndarray, gamma, alpha: np.ndarray) -> np.ndarray:
    """y = bf16(acc * gamma * alpha / 127) as uint16 bit patterns."""
    acc = _c(acc, np.int32)
    alpha = _c(alpha, np.float32)
    m, n = acc.shape
    y = np.empty((m, n), np.uint16)
    _load().orc_rescale(_p(acc), m, n, float(np.float32(gamma)), _p(alpha), _p(y))
    return y


def bitlinear_forward(packed: np.ndarray, gamma, x_bf16: np.ndarray, n: int):
    """Whole layer from packed weights: returns (y bf16 bits, acc, xq, alpha)."""
    packed = _c(packed, np.uint8)
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    alpha = np.empty(m, np.float32)
    acc = np.empty((m, n), np.int32)
    y = np.empty((m, n), np.uint16)
    rc = _load().orc_bitlinear_forward(_p(packed), float(np.float32(gamma)), _p(x), m, n, k,
                                       _p(xq), _p(alpha), _p(acc), _p(y))
    if rc != 0:
        raise ValueError("k must be a multiple of 64")
    return y, acc, xq, alpha


def glu(acc: np.ndarray, gamma, alpha: np.ndarray) -> np.ndarray:
    """Squared-ReLU gating of a gate+up product: acc [m][2f] (gate rows, then
    up rows) -> h [m][f] bf16 bits, h = relu(g)^2 * u from the exact rescaled
    values, rounded once."""
    acc = _c(acc, np.int32)
    alpha = _c(alpha, np.float32)
    m, n2 = acc.shape
    assert n2 % 2 == 0
    h = np.empty((m, n2 // 2), np.uint16)
    _load().orc_glu(_p(acc), m, n2 // 2, float(np.float32(gamma)), _p(alpha), _p(h))
    return h


def pack_glu(q: np.ndarray) -> np.ndarray:
    """Pack a gate+up ternary matrix [2f][k] with alternating gate/up 16-row tiles."""
    q = _c(q, np.int8)
    n2, k = q.shape
    out = np.empty(packed_bytes(n2, k), np.uint8)
    rc = _load().orc_pack_glu(_p(q), n2 // 2, k, _p(out))
    if rc != 0 or n2 % 2:
        raise ValueError(f"orc_pack_glu failed ({rc})")
    return out


def unpack_glu(packed: np.ndarray, f: int, k: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    if packed.size != packed_bytes(2 * f, k):
        raise ValueError("packed buffer has the wrong size")
    q = np.empty((2 * f, k), np.int8)
    rc = _load().orc_unpack_glu(_p(packed), f, k, _p(q))
    if rc != 0:
        raise ValueError(f"orc_unpack_glu failed ({rc})")
    return q


def ternarize_pack_glu(w: np.ndarray):
    """Gate+up weights [2f][k] -> (packed in the alternating order, gamma of the whole matrix)."""
    g = absmean(w)
    return pack_glu(ternarize(w, g)), g


def bitlinear_glu_forward(packed: np.ndarray, gamma, x_bf16: np.ndarray, f: int):
    """Quantize, gate+up product from the alternating packing, squared-ReLU
    gating: returns (h bf16 bits [m][f], acc [m][2f], xq, alpha)."""
    packed = _c(packed, np.uint8)
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    alpha = np.empty(m, np.float32)
    acc = np.empty((m, 2 * f), np.int32)
    h = np.empty((m, f), np.uint16)
    rc = _load().orc_bitlinear_glu_forward(_p(packed), float(np.float32(gamma)), _p(x), m, f, k,
                                           _p(xq), _p(alpha), _p(acc), _p(h))
    if rc != 0:
        raise ValueError("k must be a multiple of 64 and f of 16")
    return h, acc, xq, alpha


def backward_x(packed: np.ndarray, gamma, dy_bf16: np.ndarray, n: int, k: int) -> np.ndarray:
    """Straight-through input gradient: dx[i][t] = gamma * sum_j dy[i][j] * q[j][t] (fp32 [m][k])."""
    packed = _c(packed, np.uint8)
    dy = _c(dy_bf16, np.uint16)
    m = dy.shape[0]
    assert dy.shape[1] == n
    dx = np.empty((m, k), np.float32)
    if _load().orc_backward_x(_p(packed), float(np.float32(gamma)), _p(dy), m, n, k, _p(dx)) != 0:
        raise ValueError("k must be a multiple of 64")
    return dx


def backward_w(dy_bf16: np.ndarray, qx: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """Straight-through weight gradient: dw[j][t] = sum_i dy[i][j] * alpha_i * qx[i][t] / 127 (fp32 [n][k])."""
    dy = _c(dy_bf16, np.uint16)
    qx = _c(qx, np.int8)
    alpha = _c(alpha, np.float32)
    m, n = dy.shape
    k = qx.shape[1]
    assert qx.shape[0] == m and alpha.shape == (m,)
    dw = np.empty((n, k), np.float32)
    _load().orc_backward_w(_p(dy), _p(qx), _p(alpha), m, n, k, _p(dw))
    return dw


def pack_transposed(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    """Packed q^T ([k][n], n % 64 == 0) from packed q ([n][k])."""
    packed = _c(packed, np.uint8)
    out = np.empty(packed_bytes(k, n), np.uint8)
    rc = _load().orc_pack_transposed(_p(packed), n, k, _p(out))
    if rc != 0:
        raise ValueError(f"orc_pack_transposed failed ({rc})")
    return out


def packed_bytes_b3(n: int, k: int) -> int:
    """Size of the five-trits-per-byte buffer: ceil(n/16)*16 rows of ceil(k/320)*64 bytes."""
    return int(_load().orc_packed_bytes_b3(n, k))


def b3_encode(trits) -> int:
    """The byte of five trits (t_0 most significant base-3 digit)."""
    t = _c(trits, np.int8)
    assert t.shape == (5,)
    return int(_load().orc_b3_encode(_p(t)))


def b3_decode(byte: int):
    """The five trits of a byte, or None if the byte is no code."""
    t = np.empty(5, np.int8)
    if _load().orc_b3_decode(int(byte), _p(t)) != 0:
        return None
    return t


def pack_b3(q: np.ndarray) -> np.ndarray:
    """Pack a ternary matrix ``[n][k]`` (k % 64 == 0) five trits per byte."""
    q = _c(q, np.int8)
    n, k = q.shape
    out = np.empty(packed_bytes_b3(n, k), np.uint8)
    rc = _load().orc_pack_b3(_p(q), n, k, _p(out))
    if rc != 0:
        raise ValueError(f"orc_pack_b3 failed ({rc})")
    return out


def unpack_b3(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    if packed.size != packed_bytes_b3(n, k):
        raise ValueError("packed buffer has the wrong size")
    q = np.empty((n, k), np.int8)
    rc = _load().orc_unpack_b3(_p(packed), n, k, _p(q))
    if rc != 0:
        raise ValueError(f"orc_unpack_b3 failed ({rc})")
    return q


def ternarize_pack_b3(w: np.ndarray):
    """Full weight preparation in the five-trits-per-byte code: (packed, gamma)."""
    g = absmean(w)
    return pack_b3(ternarize(w, g)), g


def bitlinear_forward_b3(packed: np.ndarray, gamma, x_bf16: np.ndarray, n: int):
    """Whole layer from five-trits-per-byte weights: (y bf16 bits, acc, xq, alpha)."""
    packed = _c(packed, np.uint8)
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    alpha = np.empty(m, np.float32)
    acc = np.empty((m, n), np.int32)
    y = np.empty((m, n), np.uint16)
    rc = _load().orc_bitlinear_forward_b3(_p(packed), float(np.float32(gamma)), _p(x), m, n, k,
                                          _p(xq), _p(alpha), _p(acc), _p(y))
    if rc != 0:
        raise ValueError("k must be a multiple of 64")
    return y, acc, xq, alpha


def set_threads(n: int = 0) -> int:
    """Set the OpenMP thread count of the oracle's loops (0: leave it);
    returns the count now in effect."""
    return int(_load().orc_set_threads(int(n)))
