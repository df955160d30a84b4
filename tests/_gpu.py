"""Helpers for the GPU parity tests: numpy <-> device tensors, comparisons."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = torch.device("cuda", 0)


def say(msg: str) -> None:
    """Name the case before a GPU step, so a crash still tells which one ran."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def i8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int8)).to(DEV)


def u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bf16_within_one_ulp(got_bits: np.ndarray, want_bits: np.ndarray) -> None:
    """|got - want| <= one bf16 ulp of want's binade (relative <= 2^-7 = 7.8e-3);
    an exact zero must stay zero."""
    got = bf16_bits_to_f64(got_bits)
    want = bf16_bits_to_f64(want_bits)
    assert got.shape == want.shape
    zero = want == 0
    assert (got[zero] == 0).all(), "acc = 0 must give exactly 0"
    nz = ~zero
    _, e = np.frexp(np.abs(want[nz]))
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    err = np.abs(got[nz] - want[nz])
    bad = err > ulp
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outputs differ by more than one bf16 ulp; "
                           f"worst relative {np.max(err / np.abs(want[nz])):.3e}")
