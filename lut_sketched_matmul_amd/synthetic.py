"""Seeded synthetic inputs for the sketched-weight matmul.

This module only draws random numbers and stores them in the tensor formats the
library consumes. It holds none of the method's arithmetic: no unpacking, no
dequantisation, no matmul, no binning. The CPU oracle and the HIP path both
take their inputs from here, so both sides see the same bits.

Formats (the library's data layout):
  * ``idx_packed``: uint8 ``[n][d*b/8]``. The b-bit indices of one row form a
    little-endian bitstream (field j occupies bits ``b*j .. b*j+b-1``, bit p
    of the stream is bit ``p % 8`` of byte ``p // 8``). Indices that are
    i.i.d. uniform in ``[0, 2^b)`` make every bit of that stream an independent
    fair coin, so uniform random bytes *are* uniformly drawn packed indices;
    nothing has to be packed here.
  * ``lut``: ``[n][gpr][2^b]`` per (row, group) lookup tables. Each table is
    ``2^b`` i.i.d. draws from a zero-mean normal with the given standard
    deviation, sorted ascending, then rounded to the storage dtype.
  * activations ``X [m][d]`` and output gradients ``dY [m][n]``.

bf16 has no numpy dtype; bf16 tensors are returned as ``uint16`` bit patterns
(round-to-nearest-even from float32) and tagged by the caller's dtype string.
"""
from __future__ import annotations

import zlib

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def rng_for(name: str) -> np.random.Generator:
    """PCG64 generator seeded with crc32 of a descriptive tensor name."""
    return np.random.Generator(np.random.PCG64(zlib.crc32(name.encode("utf-8"))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to a storage dtype: f32, f16 (numpy RNE) or bf16 bits."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float32).astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored tensor (every f32/f16/bf16 value is exact in f64)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x).astype(np.float64)


def packed_row_bytes(d: int, b: int) -> int:
    if (d * b) % 8:
        raise ValueError(f"d*b must be a multiple of 8 (d={d}, b={b})")
    return d * b // 8


def random_packed_indices(name: str, n: int, d: int, b: int) -> np.ndarray:
    """Uniform i.i.d. b-bit indices, already in the packed little-endian layout."""
    nb = packed_row_bytes(d, b)
    g = rng_for(name)
    return g.integers(0, 256, size=(n, nb), dtype=np.uint8)


def random_lut(name: str, n: int, gpr: int, b: int, sigma: float, dtype: str) -> np.ndarray:
    """Sorted N(0, sigma) tables, one per (row, group), stored in ``dtype``."""
    k = 1 << b
    g = rng_for(name)
    draws = g.standard_normal(size=(n, gpr, k), dtype=np.float32) * np.float32(sigma)
    draws.sort(axis=-1)
    return to_storage(draws, dtype)


def random_normal(name: str, shape, sigma: float, dtype: str) -> np.ndarray:
    """i.i.d. N(0, sigma) tensor stored in ``dtype``."""
    g = rng_for(name)
    x = g.standard_normal(size=tuple(shape), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return to_storage(x, dtype)


def random_int_valued(name: str, shape, lo: int, hi: int, dtype: str) -> np.ndarray:
    """Integers uniform in ``[lo, hi]`` stored in ``dtype`` (exact for |v| <= 256)."""
    g = rng_for(name)
    x = g.integers(lo, hi + 1, size=tuple(shape)).astype(np.float32)
    return to_storage(x, dtype)
