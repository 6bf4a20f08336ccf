"""Bit packing and fp16 storage helpers.

Hub, "technical principle", step 5: 2-bit codes are packed four to a byte and
4-bit codes two to a byte.  Reading (the pages fix neither the bit order nor
3-bit packing): every packed field is a little-endian, LSB-first bit stream —
element j of a b-bit field occupies stream bits [b*j, b*j + b), and stream
bit i is bit (i mod 8) of byte (i div 8).  At 2 and 4 bits this is exactly the
pages' 4-per-byte / 2-per-byte packing; at 3 bits it is a dense stream of
8 codes per 3 bytes.  A QJL sign bit is a 1-bit field.

Metadata (norms, scales, zero-points) is stored as IEEE binary16 with
round-to-nearest-even (reading: the iThome article only says norm, scale and
zero-point metadata is stored, not its type).
"""

from __future__ import annotations

import numpy as np

__all__ = ["pack", "unpack", "to_fp16_bits", "from_fp16_bits"]


def pack(values, b: int) -> np.ndarray:
    """Pack non-negative integers < 2**b along the last axis into bytes."""
    v = np.asarray(values, dtype=np.int64)
    if np.any(v < 0) or np.any(v >= (1 << b)):
        raise ValueError("value out of range for the bit width")
    m = v.shape[-1]
    if (m * b) % 8:
        raise ValueError("field does not fill whole bytes")
    # bit k of element j -> stream bit b*j + k
    bitplanes = ((v[..., :, None] >> np.arange(b)) & 1).astype(np.uint8)
    stream = bitplanes.reshape(v.shape[:-1] + (m * b,))
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack(packed, b: int, m: int) -> np.ndarray:
    """Inverse of :func:`pack`: ``m`` b-bit integers from each row of bytes."""
    p = np.asarray(packed, dtype=np.uint8)
    stream = np.unpackbits(p, axis=-1, bitorder="little")[..., : m * b]
    planes = stream.reshape(p.shape[:-1] + (m, b))
    out = np.zeros(p.shape[:-1] + (m,), dtype=np.uint16 if b > 8 else np.uint8)
    for k in range(b):  # stream bit b*j + k is bit k of element j
        out |= planes[..., k].astype(out.dtype) << k
    return out.astype(np.int64)


def to_fp16_bits(x) -> np.ndarray:
    """binary16 bit patterns (uint16) of x rounded to nearest even."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def from_fp16_bits(h) -> np.ndarray:
    """fp64 values of binary16 bit patterns."""
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)
