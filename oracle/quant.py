"""Front-end quantisers of one DSA layer step, as a plain NumPy reference.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this package; the product path never imports it.

What they follow (Kimi K3.1 Pro day-0 page, "Low-latency decoding: the fused
DSA decode path"): the indexer front end quantises the index query to FP8 or
MXFP4 with the head weights folded into the quantisation, and writes the new
token's index key; the MLA query step writes the new token's latent into the
KV cache.  Cache formats: same page, "One KV cache, three states", and the AMD
section "native MXFP4 indexer".  Scale rules (the plainest reading where the
pages give none; the readings table lists them):

  FP8 row    s = amax / 448 (1 for an all-zero row); code = E4M3(x / s)
  MXFP4      per 32 values X = floor(log2 amax) - 2, read from amax's fp32
             exponent field; E8M0 code = X + 127 clamped to 0..254;
             code = E2M1(x / 2^(E8M0 - 127))
  NVFP4      per 16 values s = E4M3(amax / 6); code = E2M1(x / value(s)),
             0 when s decodes to 0; rope dims E4M3(x), unscaled (latents);
             index keys the same rule over their 128 dims (MiniMax-M3.1 page,
             "Quick start": NVFP4 index keys)
  folding    FP8 query rows: w' = w * s, so that w' * ReLU(code . k) equals
             w * ReLU((s * code) . k) for s > 0 (ReLU is positively
             homogeneous)

E4M3 and E2M1 codes are the nearest representable value, ties to the even
code, saturating (448 and 6); a result of zero is stored as +0.  Every
division that decides a code is taken in fp32 -- the precision the kernels
use -- and the code is then the exact rounding of that fp32 value (computed in
fp64, where the rounding below is exact).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> fp32 values (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# ---------------------------------------------------------------- element codes
def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3FN codes (uint8), nearest even, saturating at 448."""
    v = f32(v)
    a = np.minimum(np.abs(v.astype(np.float64)), E4M3_MAX)
    tiny = a < 2.0 ** -6  # below the smallest normal: multiples of 2^-9
    sub_units = np.rint(a * 2.0 ** 9)  # exact product, ties to even; 8 = 2^-6
    m, e = np.frexp(np.where(tiny, 1.0, a))  # a = m 2^e, 1/2 <= m < 1
    e = e - 1
    frac = np.rint((2.0 * m - 1.0) * 8.0)  # mantissa in eighths, ties to even
    carry = frac == 8.0
    e = e + carry
    frac = np.where(carry, 0.0, frac)
    normal = (e.astype(np.int64) + 7) * 8 + frac.astype(np.int64)
    code = np.where(tiny, sub_units.astype(np.int64), normal)
    neg = np.signbit(v) & (code != 0)
    return (code + 128 * neg).astype(np.uint8)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """fp32 values -> 4-bit E2M1 codes (uint8 0..15), nearest even, saturating
    at 6; code c is magnitude E2M1_MAGS[c & 7], sign bit 8."""
    v = f32(v)
    a = np.minimum(np.abs(v.astype(np.float64)), E2M1_MAX)
    lo = np.searchsorted(E2M1_MAGS, a, side="right") - 1  # largest code at or below a
    hi = np.minimum(lo + 1, 7)
    d_lo = a - E2M1_MAGS[lo]
    d_hi = E2M1_MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    neg = np.signbit(v) & (code != 0)
    return (code + 8 * neg).astype(np.uint8)


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes -> fp32 values (finite codes only)."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return f32(s * mag)


def pack_pairs(nib: np.ndarray) -> np.ndarray:
    """[..., 2n] 4-bit codes -> [..., n] bytes, element 2i in the low nibble."""
    nib = np.asarray(nib).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------- block rules
def fp8_row(x: np.ndarray):
    """FP8 row quantisation along the last axis.  Returns (codes uint8 [..., d],
    scale fp32 [...])."""
    x = f32(x)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, f32(amax / f32(E4M3_MAX)), f32(1.0)).astype(np.float32)
    y = f32(x / scale[..., None])
    return e4m3_encode(y), scale


def mx_e8m0(amax: np.ndarray) -> np.ndarray:
    """E8M0 code of an MX block: floor(log2 amax) - 2 + 127 from the fp32
    exponent field of amax, clamped to 0..254."""
    field = (f32(amax).view(np.uint32) >> 23) & 0xFF
    return np.clip(field.astype(np.int64) - 127 - 2 + 127, 0, 254).astype(np.uint8)


def mxfp4_blocks(x: np.ndarray, block: int = 32):
    """MXFP4 along the last axis.  Returns (packed codes uint8 [..., d/2],
    E8M0 codes uint8 [..., d/block])."""
    x = f32(x)
    xb = x.reshape(*x.shape[:-1], x.shape[-1] // block, block)
    e8 = mx_e8m0(np.abs(xb).max(axis=-1))
    scale = f32(np.exp2(e8.astype(np.float64) - 127.0))
    y = f32(xb / scale[..., None])
    return pack_pairs(e2m1_encode(y).reshape(x.shape)), e8


def nvfp4_blocks(x: np.ndarray, block: int = 16):
    """NVFP4 along the last axis.  Returns (packed codes uint8 [..., d/2],
    E4M3 block-scale codes uint8 [..., d/block])."""
    x = f32(x)
    xb = x.reshape(*x.shape[:-1], x.shape[-1] // block, block)
    sc = e4m3_encode(f32(np.abs(xb).max(axis=-1) / f32(E2M1_MAX)))
    sv = e4m3_value(sc)
    safe = np.where(sv > 0, sv, f32(1.0)).astype(np.float32)
    nib = e2m1_encode(f32(xb / safe[..., None]))
    nib = np.where((sv > 0)[..., None], nib, 0).astype(np.uint8)
    return pack_pairs(nib.reshape(x.shape)), sc


# ---------------------------------------------------------------- entry points
def quantize_q(q_bits: np.ndarray, w: np.ndarray | None, fmt: str):
    """Index-query quantisation per (row, head).  q_bits: bf16 bits [T, 32, 128].
    FP8: returns (codes [T,32,128], scale fp32 [T,32], w_folded fp32 [T,32] or
    None).  MXFP4: returns (packed codes [T,32,64], E8M0 [T,32,4], None)."""
    q = bf16_to_f32(q_bits)
    if fmt == "fp8":
        codes, scale = fp8_row(q)
        wf = None if w is None else f32(f32(w) * scale)
        return codes, scale, wf
    if fmt == "mxfp4":
        codes, e8 = mxfp4_blocks(q, 32)
        return codes, e8, None
    raise ValueError(fmt)


KEY_CODE_BYTES = {"fp8": 128, "mxfp4": 64, "nvfp4": 64}
KEY_SIDE_BYTES = {"fp8": 4, "mxfp4": 4, "nvfp4": 8}
LAT_ROW_STRIDE = {"bf16": 1152, "fp8": 640, "nvfp4": 384}


def insert_key(pool: np.ndarray, fmt: str, P: int, page: int, slot: int, vals_bits: np.ndarray):
    """Write one token's index key (bf16 bits [128]) into page `page`, slot
    `slot` of a key pool [pages, page_bytes] (in place)."""
    x = bf16_to_f32(vals_bits)
    cb, sb = KEY_CODE_BYTES[fmt], KEY_SIDE_BYTES[fmt]
    if fmt == "fp8":
        codes, scale = fp8_row(x)
        side = np.asarray([scale], np.float32).view(np.uint8)
    elif fmt == "mxfp4":
        codes, side = mxfp4_blocks(x, 32)
    else:
        codes, side = nvfp4_blocks(x, 16)
    pool[page, slot * cb:(slot + 1) * cb] = codes
    pool[page, P * cb + slot * sb:P * cb + (slot + 1) * sb] = side


def insert_latent(pool: np.ndarray, fmt: str, P: int, page: int, slot: int, vals_bits: np.ndarray):
    """Write one token's latent (bf16 bits [576]) into its row (in place);
    the row's unused tail bytes are left as they are."""
    x = bf16_to_f32(vals_bits)
    base = slot * LAT_ROW_STRIDE[fmt]
    row = pool[page]
    if fmt == "bf16":
        row[base:base + 1152] = np.asarray(vals_bits).astype(np.uint16).view(np.uint8)
    elif fmt == "fp8":
        codes, scale = fp8_row(x)
        row[base:base + 576] = codes
        row[base + 576:base + 580] = np.asarray([scale], np.float32).view(np.uint8)
    else:
        codes, sc = nvfp4_blocks(x[:512], 16)
        row[base:base + 256] = codes
        row[base + 256:base + 288] = sc
        row[base + 288:base + 352] = e4m3_encode(x[512:])


def cache_insert(key_pool, key_fmt, lat_pool, lat_fmt, P, block_table, tok_req, tok_pos, key_bits, lat_bits,
                 num_pages):
    """Insert n new tokens (request tok_req[i], position tok_pos[i]) into copies
    of the pools; a token whose page lookup falls outside the table or the
    pool is skipped.  Returns (key_pool, lat_pool)."""
    kp = None if key_pool is None else key_pool.copy()
    lp = None if lat_pool is None else lat_pool.copy()
    for i in range(len(tok_req)):
        r, pos = int(tok_req[i]), int(tok_pos[i])
        lpg = pos // P
        if block_table is None:
            page = r
        else:
            if pos < 0 or lpg >= block_table.shape[1]:
                continue
            page = int(block_table[r, lpg])
        if page < 0 or page >= num_pages or pos < 0:
            continue
        if kp is not None and key_bits is not None:
            insert_key(kp, key_fmt, P, page, pos % P, key_bits[i])
        if lp is not None and lat_bits is not None:
            insert_latent(lp, lat_fmt, P, page, pos % P, lat_bits[i])
    return kp, lp
