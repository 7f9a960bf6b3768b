"""Algorithmic bytes and flops of one DSA layer step (what the method must move
and compute, not what a given kernel happens to move).

Per-token widths (Kimi K3.1 Pro day-0 page, "One KV cache, three states"):
FP8 index key 132 B (128 values + fp32 scale), MXFP4 index key 68 B, FP8
latent 576 B (+ a 4-byte per-token scale in this layout = 580 B), NVFP4 latent
352 B, BF16 latent 1152 B; NVFP4 index key 72 B (64 B of E2M1 pairs + 8 E4M3
block scales; MiniMax-M3.1 page, "Quick start").

Counted per step:
  * index keys once per request (speculative rows of a request share them;
    AMD section "native MXFP4 indexer"): max_vis(r) x key bytes;
  * K_t = min(k, vis_t) latent rows per query row;
  * small terms: indexer q and w, MLA q, outputs (fp32 o + lse), block table.
Not counted: the fp32 score round trip between indexer and top-k, and split
partials, which are artefacts of the kernel split (reported separately).

Flops: indexer 2 x 32 x 128 per visible (row, key) pair; MLA
2 x H x K_t x (576 + 512) per row (real heads, not padded).
"""
from __future__ import annotations

KEY_B = {"fp8": 132, "mxfp4": 68, "nvfp4": 72}
LAT_B = {"bf16": 1152, "fp8": 580, "nvfp4": 352}
LAT_B_PAGE_FORMULA = {"bf16": 1152, "fp8": 576, "nvfp4": 352}
HBM_PEAK = 8.0e12           # B/s, MI355X (MI355X Kimi K3 page, introduction)
TOPK = 2048                 # tokens kept per query ("Sparse attention in K3.1 Pro")


def step_bytes(*, req_vis_max, row_vis, k, H, key_fmt, lat_fmt, q_fmt="bf16", page=64):
    """Dict of algorithmic byte terms for one step.

    req_vis_max: visible keys of each request's last row; row_vis: per row."""
    keys = sum(int(n) * KEY_B[key_fmt] for n in req_vis_max)
    K = [min(k, int(v)) for v in row_vis]
    lat = sum(K) * LAT_B[lat_fmt]
    T = len(row_vis)
    q_idx = T * (32 * 128 * 2 if q_fmt == "bf16" else 32 * 128 + 32 * 4)
    w = T * 32 * 4
    q_mla = T * H * 576 * 2
    outs = T * H * (512 * 4 + 4)
    bt = 0 if page == 0 else sum((int(n) + page - 1) // page * 4 for n in req_vis_max)
    small = q_idx + w + q_mla + outs + bt
    return {"keys": keys, "latents": lat, "small": small, "total": keys + lat + small,
            "indexer": keys + q_idx + w + bt, "mla": lat + q_mla + outs}


def step_flops(*, row_vis, k, H):
    idx = sum(int(v) for v in row_vis) * 2 * 32 * 128
    mla = sum(min(k, int(v)) for v in row_vis) * 2 * H * (576 + 512)
    return {"indexer": idx, "mla": mla}


def literal_formula_bytes(queries: int, N: int, k: int = 2048) -> int:
    """queries * (N * 132 + k * 576): the FP8 byte formula quoted for decode."""
    return queries * (N * 132 + k * 576)


def dense_vs_sparse_ratio(N: int, k: int = 2048) -> float:
    """Bytes of a DSA decode step over dense MLA's at context N, one query,
    FP8 (Kimi K3.1 Pro day-0 page, "Sparse attention in K3.1 Pro": about 23%)."""
    return (N * 132 + min(k, N) * 576) / (N * 576)


def index_key_saving(fmt_from: str, fmt_to: str) -> float:
    """Fraction of index-cache storage saved by switching key formats (AMD
    "native MXFP4 indexer": 132 -> 68 bytes, 48.5% less)."""
    return 1.0 - KEY_B[fmt_to] / KEY_B[fmt_from]


def cache_bytes_per_token(key_fmt: str, lat_fmt: str) -> int:
    """Bytes one token holds in one layer: its latent (as the pages count it)
    plus its index key ("DCP prefill without merge": about 0.7 GB per 1M FP8
    tokens)."""
    return LAT_B_PAGE_FORMULA[lat_fmt] + KEY_B[key_fmt]


def candidate_exchange_bytes(k: int, ids: bool) -> int:
    """Bytes one rank sends per query when exchanging its k candidates: 4-byte
    scores, plus 4-byte ids when they travel too (AMD "Communication": 16 KiB
    -> 8 KiB for 2,048 candidates when only scores are exchanged)."""
    return k * (8 if ids else 4)


def latent_cache_bytes(layers: int, tokens: int, bytes_per_token: int) -> int:
    """MLA payload of a cache (MI355X Kimi K3 page, section 1 "Cache":
    24 layers x 142,000 positions x 576 B = about 1.96 GB)."""
    return layers * tokens * bytes_per_token


def padded_heads(H: int) -> int:
    """Query heads after padding to the 16-row MFMA tile (MI355X Kimi K3 page,
    section 4 "MLA": 12 -> 16)."""
    return (H + 15) // 16 * 16
