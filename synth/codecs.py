"""Encoders (real value -> storage code) for the cache formats of one DSA layer.

These only *produce* inputs.  Decoding a code back to a value is a step of the
method itself and lives separately in the oracle (fp64, NumPy) and in the HIP
kernels; neither of them imports this module's arithmetic.

Formats (byte budgets from the Kimi K3.1 Pro day-0 page, "One KV cache, three
states" and the AMD section "native MXFP4 indexer"):

* E4M3  -- OCP FP8 E4M3FN: bias 7, max finite 448, S.1111.111 is NaN.  Encoded
  round-to-nearest-even and saturated to +-448, so NaN is never written.
* E2M1  -- OCP FP4: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; two codes per byte,
  element 2i in the low nibble.  Round-to-nearest-even, saturated to +-6.
* E8M0  -- power-of-two scale 2**(code-127); 0xFF (NaN) is never written (the
  MXFP4 engineering-log page, phase-2 "NaN/Inf decision record").
* BF16  -- round-to-nearest-even from fp32 (the MI355X Kimi K3 page, KDA
  precision note: 256.5 rounds to 256).
"""
from __future__ import annotations

import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 (RNE) returned as a torch.bfloat16 tensor."""
    return x.to(torch.float32).to(torch.bfloat16)


def e4m3_encode(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> uint8 E4M3FN codes, RNE, saturating to +-448."""
    x = x.to(torch.float32).clamp(-E4M3_MAX, E4M3_MAX)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def e4m3_value(codes: torch.Tensor) -> torch.Tensor:
    """uint8 E4M3FN codes -> fp32 (generator-side only: used to divide by a
    stored block scale when quantising NVFP4 elements)."""
    return codes.view(torch.float8_e4m3fn).to(torch.float32)


# Decision thresholds for E2M1 round-to-nearest-even on the magnitude.  At a
# midpoint the code with the even mantissa bit wins, so some comparisons are
# strict and some are not.
_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_TIE_UP = (False, True, False, True, False, True, False)


def e2m1_encode_nibbles(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> uint8 tensor of 4-bit E2M1 codes (one code per element, 0..15)."""
    x = x.to(torch.float32)
    mag = x.abs().clamp(max=E2M1_MAX)
    code = torch.zeros_like(mag, dtype=torch.uint8)
    for mid, up in zip(_E2M1_MIDS, _E2M1_TIE_UP):
        code += (mag >= mid if up else mag > mid).to(torch.uint8)
    sign = (torch.signbit(x) & (code != 0)).to(torch.uint8)
    return code | (sign << 3)


def pack_nibbles(nib: torch.Tensor) -> torch.Tensor:
    """[..., 2n] 4-bit codes -> [..., n] bytes, element 2i in the low nibble."""
    lo = nib[..., 0::2]
    hi = nib[..., 1::2]
    return (lo | (hi << 4)).to(torch.uint8)


def fp8_rowwise(x: torch.Tensor):
    """Per-row FP8: scale = amax/448 (fp32), codes = E4M3(x/scale).

    Returns (codes uint8 [..., d], scale fp32 [...]).  An all-zero row gets
    scale 1 so that it decodes to zeros."""
    x = x.to(torch.float32)
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = e4m3_encode(x / scale.unsqueeze(-1))
    return codes, scale


def mxfp4_blocks(x: torch.Tensor, block: int = 32):
    """OCP MX FP4 quantisation along the last dim.

    Shared exponent X = floor(log2(amax)) - 2 (2 is E2M1's largest exponent),
    stored as E8M0 code X+127 and clamped to 0..254; elements are E2M1(x/2**X).
    Returns (packed codes uint8 [..., d/2], e8m0 uint8 [..., d/block])."""
    x = x.to(torch.float32)
    shp = x.shape
    xb = x.reshape(*shp[:-1], shp[-1] // block, block)
    amax = xb.abs().amax(dim=-1)
    # floor(log2(amax)) from the fp32 exponent field (exact, no log rounding)
    bits = amax.view(torch.int32)
    expo = ((bits >> 23) & 0xFF) - 127
    X = torch.where(amax > 0, expo - 2, torch.full_like(expo, -127))
    code = (X + 127).clamp(0, 254)
    scale = torch.ldexp(torch.ones_like(amax), (code - 127).to(torch.int32))
    nib = e2m1_encode_nibbles(xb / scale.unsqueeze(-1)).reshape(shp)
    return pack_nibbles(nib), code.to(torch.uint8)


def nvfp4_blocks(x: torch.Tensor, block: int = 16):
    """NVFP4 quantisation along the last dim: per-16 scale E4M3(amax/6),
    elements E2M1(x/scale) saturating.  Returns (packed uint8 [..., d/2],
    scale codes uint8 [..., d/block])."""
    x = x.to(torch.float32)
    shp = x.shape
    xb = x.reshape(*shp[:-1], shp[-1] // block, block)
    amax = xb.abs().amax(dim=-1)
    sc = e4m3_encode(amax / E2M1_MAX)
    sv = e4m3_value(sc)
    safe = torch.where(sv > 0, sv, torch.ones_like(sv))
    nib = e2m1_encode_nibbles(xb / safe.unsqueeze(-1))
    nib = torch.where((sv > 0).unsqueeze(-1), nib, torch.zeros_like(nib))
    return pack_nibbles(nib.reshape(shp)), sc
