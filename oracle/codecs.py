"""Oracle-side decoders: storage code -> exact value (fp64), written from the
format definitions.  TEST INFRASTRUCTURE ONLY -- see oracle/__init__.py.

* E4M3FN (OCP FP8): sign | 4-bit exponent (bias 7) | 3-bit mantissa.  Exponent
  0 is subnormal (m * 2**-9); code S.1111.111 is NaN; max finite 448.
* E2M1 (OCP FP4): sign | 2-bit exponent (bias 1) | 1-bit mantissa; the eight
  magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} (MiniMax-M3.1 day-0 page, AMD section
  "NVFP4 MSA kernels": 8 E2M1 magnitudes).  Element 2i of a byte pair sits in
  the low nibble (the MXFP4 engineering-log page, phase 1: two FP4 per byte).
* E8M0: 2**(code-127); 0xFF is NaN (MXFP4 engineering-log page, phase 2
  "NaN/Inf decision record").
* BF16: the upper half of an IEEE binary32.
"""
from __future__ import annotations

import math

import numpy as np


def _e4m3_value(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _e2m1_value(c: int) -> float:
    s = -1.0 if c & 0x8 else 1.0
    e = (c >> 1) & 0x3
    m = c & 0x1
    if e == 0:
        return s * 0.5 * m
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([math.ldexp(1.0, c - 127) if c != 255 else math.nan
                       for c in range(256)], dtype=np.float64)


def e4m3(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_packed(b: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] values (low nibble first)."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.float64)
    out[..., 0::2] = E2M1_TABLE[b & 0xF]
    out[..., 1::2] = E2M1_TABLE[b >> 4]
    return out


def e8m0(codes: np.ndarray) -> np.ndarray:
    return E8M0_TABLE[np.asarray(codes, dtype=np.uint8)]


def bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 (or int16) bf16 bit patterns -> fp64."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32(raw: np.ndarray) -> np.ndarray:
    """little-endian bytes [..., 4k] -> fp64 [..., k]."""
    raw = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8))
    return raw.view("<f4").astype(np.float64)
