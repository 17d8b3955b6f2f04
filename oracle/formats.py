"""Exact decoding of the stored input formats to fp64, and bf16 storage
rounding.  Test infrastructure; see package docstring.

Formats (the storage the library consumes):
* bf16 bit patterns (uint16): value = float32 with the 16 bits as its top half.
* int4 groups of 32 along the reduction axis: packed uint32 [N, K/8], nibble i
  of word m holds (code + 8) for reduction index 8m + i; bf16 scale per
  (row, group of 32); weight = code * scale (exact in fp64).
* fp32 arrays.
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_to_f64", "int4_to_f64", "matrix_f64", "round_bf16"]


def bf16_to_f64(u) -> np.ndarray:
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def int4_to_f64(packed, scales) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint32)
    n, kw = packed.shape
    codes = np.empty((n, kw, 8), dtype=np.float64)
    for i in range(8):
        codes[..., i] = ((packed >> np.uint32(4 * i)) & np.uint32(15)).astype(np.float64) - 8.0
    s = bf16_to_f64(scales)                         # [n, K/32]
    w = codes.reshape(n, kw * 8).reshape(n, -1, 32) * s[..., None]
    return w.reshape(n, kw * 8)


def matrix_f64(w, rows: slice | None = None) -> np.ndarray:
    """Decode a workloads.Weights (or a subset of its rows) to fp64 [N, K]."""
    sl = rows if rows is not None else slice(None)
    if w.wtype == "f32":
        return np.asarray(w.data[sl], dtype=np.float64)
    if w.wtype == "bf16":
        return bf16_to_f64(w.data[sl])
    if w.wtype == "int4":
        return int4_to_f64(w.data[sl], w.scale[sl])
    raise ValueError(w.wtype)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as
    fp64.  bf16 keeps 8 significant bits: write x = m * 2^e with 0.5 <= |m| < 1
    and round m * 2^8 to an integer, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)
