"""Seeded synthetic inputs, shared by the GPU path's tests/bench and the oracle's.

This module holds no arithmetic of the attention method: it draws normal
random numbers and rounds them to the storage type.  Both sides of every
parity check receive exactly the same values -- the GPU as bf16 (or fp32)
bits, the oracle as the same values upcast to float64 without rounding.

Recipe: ``numpy.random.Generator(PCG64(seed))``; arrays are drawn in the order
the caller asks for them (Q, then K, then V); each is a float32 standard
normal times a per-tensor scale, rounded once to bf16 with round-to-nearest-
even when the storage type is bf16.
"""

from __future__ import annotations

import hashlib

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the generators never produce inf or NaN).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # For finite values u + 0x8000 stays below 2**32, so uint32 cannot wrap.
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """A synthetic tensor in its storage type plus the exact float64 view.

    ``bits``: uint16 bf16 patterns (dtype "bf16") or float32 values ("f32").
    ``f64``: the same values as float64 (lazily computed, exact).
    """

    def __init__(self, storage: np.ndarray, dtype: str):
        self.storage = storage
        self.dtype = dtype

    @property
    def shape(self):
        return self.storage.shape

    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_to_f32(self.storage)
        return self.storage

    def f64(self) -> np.ndarray:
        return self.f32().astype(np.float64)

    def sha256(self) -> str:
        return hashlib.sha256(np.ascontiguousarray(self.storage).tobytes()).hexdigest()


def normal(gen: np.random.Generator, shape, scale: float, dtype: str) -> Tensor:
    """float32 N(0,1) * scale, stored as ``dtype`` ("bf16" or "f32")."""
    x = gen.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "bf16":
        return Tensor(bf16_bits(x), "bf16")
    if dtype == "f32":
        return Tensor(x, "f32")
    raise ValueError(dtype)
