"""Plain fp64 CPU definition of one DSA layer (indexer -> top-k -> sparse MLA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
it shares no code with the HIP library.  Every function is a direct, unblocked
transcription of the definition it cites; NumPy matmul/sort are the only library
steps.

Sources (page titles and sections):
  [K31]  "vLLM Day-0 support for Kimi K3.1 Pro across GPU, TPU and PPU":
         "Sparse attention in K3.1 Pro" (32 light heads score every earlier
         token, keep the top 2,048, exact MLA over those only; FP8 index key of
         132 B with its scale), "One KV cache, three states" (byte widths; block
         table -> kernel page addresses), AMD "native MXFP4 indexer" (FP32
         accumulation, weighted reduction across heads; 68 B MXFP4 keys),
         "Long context: decode context parallel" (partials merged by LSE).
  [K3]   "Optimising Kimi K3 on AMD Instinct MI355X", section 4 "MLA" (padding
         12 -> 16 query heads leaves the real heads' softmax unchanged; history
         split into parallel pieces and merged).
The pages defer the indexer formula to the DeepSeek-V3.2 article; the reading
taken here is the lightning-indexer form
    score(t, s) = sum_h w_h(t) * ReLU(q_h(t) . k_s),
with k_s the dequantised key (codes x per-token scale).  MLA latents are 576-d
(512 "nope" + 64 "rope"), V = the first 512 dims, softmax scale 1/sqrt(192).

Page layout read here (structure-of-arrays inside a key page of P tokens;
latent pages are P padded rows, see lat_rows):
  key FP8    [P x 128 E4M3][P x fp32]
  key MXFP4  [P x 64 B E2M1 pairs][P x 4 E8M0]
  key NVFP4  [P x 64 B E2M1 pairs][P x 8 E4M3 block scales, one per 16 dims]
Logical token s of request r lives in physical page bt[r][s // P], slot s % P
(non-paged caches: page r, slot s).  A physical row id is page * P + slot.

Absent pages.  A block-table entry outside [0, num_pages) names no page
("One KV cache, three states" gives the block table as the only map from a
request's tokens to pages, so such an entry maps its tokens nowhere): the
indexer scores its tokens -inf, so they rank below every present token (and
among themselves by index), and translation gives their rows -1, which
attention skips.  K_t = min(k, vis_t) is unchanged.

MiniMax-M3.1 page ("Quick start": indexer_kv_dtype nvfp4; AMD "NVFP4 indexer
DCP") keeps the index keys in NVFP4: E2M1 values with one E4M3 scale per 16
values; no second-level scale is stored here (72 B per 128-d key).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import codecs as C

HI, DI, D_LAT, D_V = 32, 128, 576, 512


# ---------------------------------------------------------------- dequantise
def key_pages(pool: np.ndarray, fmt: str, P: int, pages: np.ndarray) -> np.ndarray:
    """Dequantise whole key pages -> fp64 [len(pages)*P, 128].  Every id must
    name a page of the pool (absent pages are handled by request_keys)."""
    pages = np.asarray(pages, dtype=np.int64)
    assert np.all((pages >= 0) & (pages < pool.shape[0])), "page id outside the pool"
    pg = pool[pages]
    n = pg.shape[0]
    if fmt == "fp8":
        codes = pg[:, : 128 * P].reshape(n, P, 128)
        scale = C.f32(pg[:, 128 * P: 132 * P]).reshape(n, P)
        vals = C.e4m3(codes) * scale[..., None]
    elif fmt == "mxfp4":
        codes = pg[:, : 64 * P].reshape(n, P, 64)
        e = C.e8m0(pg[:, 64 * P: 68 * P].reshape(n, P, 4))
        vals = C.e2m1_packed(codes) * np.repeat(e, 32, axis=-1)
    elif fmt == "nvfp4":
        codes = pg[:, : 64 * P].reshape(n, P, 64)
        sc = C.e4m3(pg[:, 64 * P: 72 * P].reshape(n, P, 8))
        vals = C.e2m1_packed(codes) * np.repeat(sc, 16, axis=-1)
    else:
        raise ValueError(fmt)
    return vals.reshape(n * P, DI)


LAT_ROW_STRIDE = {"bf16": 1152, "fp8": 640, "nvfp4": 384}   # bytes per latent row in a page


def lat_rows(pool: np.ndarray, fmt: str, P: int, rows: np.ndarray) -> np.ndarray:
    """Dequantise latent rows (physical ids page*P+slot) -> fp64 [m, 576].

    A latent page holds P rows of LAT_ROW_STRIDE[fmt] bytes: BF16 [576 bf16];
    FP8 [576 E4M3][fp32 scale][pad]; NVFP4 [256 B E2M1 pairs][32 E4M3 block
    scales][64 E4M3 rope][pad] ("One KV cache, three states": 576-byte FP8 and
    352-byte NVFP4 latents; the padding is unused)."""
    rows = np.asarray(rows, dtype=np.int64)
    page, slot = rows // P, rows % P
    stride = LAT_ROW_STRIDE[fmt]

    def field(off, width):
        cols = slot[:, None] * stride + off + np.arange(width)[None, :]
        return pool[page[:, None], cols]

    if fmt == "bf16":
        return C.bf16(field(0, 1152).view("<u2"))
    if fmt == "fp8":
        return C.e4m3(field(0, 576)) * C.f32(field(576, 4))
    if fmt == "nvfp4":
        nope = C.e2m1_packed(field(0, 256))                  # [m, 512]
        sc = C.e4m3(field(256, 32))                          # [m, 32]
        rope = C.e4m3(field(288, 64))                        # [m, 64]
        return np.concatenate([nope * np.repeat(sc, 16, axis=-1), rope], axis=-1)
    raise ValueError(fmt)


def request_pages(block_table: Optional[np.ndarray], r: int, n: int, P: int,
                  num_pages: Optional[int] = None) -> np.ndarray:
    """Address translation for the scan side: logical pages 0..ceil(n/P)-1 of
    request r -> physical page ids ([K31] "One KV cache, three states"); an
    entry outside [0, num_pages) is absent and returned as -1."""
    npg = (n + P - 1) // P
    if block_table is None:
        assert npg == 1, "non-paged cache holds a request in one page"
        pages = np.array([r], dtype=np.int64)
    else:
        pages = np.asarray(block_table[r, :npg], dtype=np.int64)
    if num_pages is not None:
        pages = np.where((pages >= 0) & (pages < num_pages), pages, -1)
    return pages


def request_keys(pool, fmt, P, block_table, r, n, with_present: bool = False):
    """Dequantised keys of logical tokens 0..n-1 of request r, fp64 [n, 128].
    Tokens on an absent page read as zeros; with_present=True also returns the
    bool mask [n] of tokens whose page is present."""
    pages = request_pages(block_table, r, n, P, num_pages=pool.shape[0])
    ok = pages >= 0
    keys = np.zeros((pages.shape[0] * P, DI))
    if ok.any():
        keys.reshape(pages.shape[0], P, DI)[ok] = key_pages(pool, fmt, P, pages[ok]).reshape(-1, P, DI)
    present = np.repeat(ok, P)[:n]
    return (keys[:n], present) if with_present else keys[:n]


def translate(idx: np.ndarray, block_table: Optional[np.ndarray], r: int, P: int,
              num_pages: Optional[int] = None) -> np.ndarray:
    """Selected logical indices -> physical rows page*P + slot; -1 stays -1,
    and so does an index whose page is absent (outside [0, num_pages))."""
    idx = np.asarray(idx, dtype=np.int64)
    out = np.full(idx.shape, -1, dtype=np.int64)
    ok = idx >= 0
    li = idx[ok]
    page = np.full(li.shape, r, dtype=np.int64) if block_table is None \
        else np.asarray(block_table[r], dtype=np.int64)[li // P]
    row = page * P + li % P
    if num_pages is not None:
        row = np.where((page >= 0) & (page < num_pages), row, -1)
    out[ok] = row
    return out


# ---------------------------------------------------------------- indexer
def indexer_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """score_s = sum_h w_h * max(0, q_h . k_s) for every key row s.

    q [32,128] fp64, w [32], keys [n,128] -> [n] fp64."""
    dots = keys @ q.T                 # [n, 32]
    return np.maximum(dots, 0.0) @ w


# ---------------------------------------------------------------- top-k
def topk(scores: np.ndarray, k: int):
    """The min(k, n) highest scores, ties to the lower index; returns the
    selected indices in ascending order and tau, the score of the last one
    selected (rank min(k,n) in (score desc, index asc) order)."""
    n = scores.shape[0]
    m = min(k, n)
    if m == 0:
        return np.zeros(0, dtype=np.int64), math.inf
    order = np.lexsort((np.arange(n), -scores))
    sel = np.sort(order[:m])
    return sel, float(scores[order[m - 1]])


# ---------------------------------------------------------------- sparse MLA
def sparse_mla(q: np.ndarray, lat: np.ndarray, sm_scale: float):
    """Exact attention of every head over the given latent rows.

    q [H,576], lat [m,576] -> o [H,512], lse [H] (natural log).  No rows:
    o = 0, lse = -inf."""
    H = q.shape[0]
    if lat.shape[0] == 0:
        return np.zeros((H, D_V)), np.full(H, -math.inf)
    logits = sm_scale * (q @ lat.T)                      # [H, m]
    mx = logits.max(axis=1)
    e = np.exp(logits - mx[:, None])
    z = e.sum(axis=1)
    o = (e @ lat[:, :D_V]) / z[:, None]
    return o, mx + np.log(z)


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge partial results of disjoint row subsets ([K31] "Long context:
    decode context parallel"): lse = log sum exp(lse_i),
    o = sum exp(lse_i - lse) o_i.  Empty parts (lse = -inf) drop out."""
    mx = np.max(lse_parts, axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    wts = np.exp(lse_parts - safe[None])
    z = wts.sum(axis=0)
    lse = np.where(z > 0, safe + np.log(np.where(z > 0, z, 1.0)), -math.inf)
    o = np.einsum("sh,shd->hd", wts, o_parts) / np.where(z > 0, z, 1.0)[:, None]
    return o, lse


def dense_mla(q: np.ndarray, lat_all: np.ndarray, sm_scale: float):
    """Dense MLA over every row given (no index list)."""
    return sparse_mla(q, lat_all, sm_scale)


# ---------------------------------------------------------------- one layer
def dequant_q_idx(inp: dict, t: int) -> np.ndarray:
    """Index query of row t as fp64 [32, 128]: BF16; FP8 codes x the per-head
    fp32 scale; or MXFP4 (E2M1 pairs [32, 64] x 2^(E8M0 - 127) per 32 dims,
    scales uint8 [32, 4]) -- the quantised query forms of [K31] "Low-latency
    decoding: the fused DSA decode path" and AMD "native MXFP4 indexer"."""
    if inp["q_fmt"] == "bf16":
        return C.bf16(inp["q_idx"][t])
    if inp["q_fmt"] == "fp8":
        return C.e4m3(inp["q_idx"][t]) * np.asarray(inp["q_idx_scale"][t], np.float64)[:, None]
    if inp["q_fmt"] == "mxfp4":
        e = C.e8m0(inp["q_idx_scale"][t])                       # [32, 4]
        return C.e2m1_packed(inp["q_idx"][t]) * np.repeat(e, 32, axis=-1)
    raise ValueError(inp["q_fmt"])


def layer(inp: dict, k: int = 2048, tokens=None, want_scores: bool = True):
    """Run indexer -> top-k -> translation -> sparse MLA for the query rows in
    `tokens` (default: all).  `inp` holds NumPy arrays:

      P, key_fmt, lat_fmt, q_fmt, sm_scale, req_token_start [R+1],
      tok_vis [T], block_table [R, pages] or None, key_pool, lat_pool,
      q_idx (bf16 bits uint16 [T,32,128] or E4M3 codes), q_idx_scale [T,32],
      w [T,32], q_mla (bf16 bits uint16 [T,H,576]).

    Returns a dict with per-row lists: scores, idx (ascending), tau, rows,
    o [H,512], lse [H]."""
    rts = np.asarray(inp["req_token_start"], dtype=np.int64)
    vis = np.asarray(inp["tok_vis"], dtype=np.int64)
    T = vis.shape[0]
    tok_req = np.searchsorted(rts, np.arange(T), side="right") - 1
    tokens = range(T) if tokens is None else tokens
    P, bt = inp["P"], inp["block_table"]
    out = {"t": [], "scores": [], "idx": [], "tau": [], "rows": [], "o": [], "lse": []}
    key_cache = {}
    for t in tokens:
        r, n = int(tok_req[t]), int(vis[t])
        if r not in key_cache or key_cache[r][0].shape[0] < n:
            key_cache.clear()
            nmax = int(vis[rts[r]:rts[r + 1]].max())
            key_cache[r] = request_keys(inp["key_pool"], inp["key_fmt"], P, bt, r, nmax, with_present=True)
        keys, present = key_cache[r][0][:n], key_cache[r][1][:n]
        sc = indexer_scores(dequant_q_idx(inp, t), np.asarray(inp["w"][t], np.float64), keys)
        sc = np.where(present, sc, -math.inf)
        sel, tau = topk(sc, k)
        rows = translate(sel, bt, r, P, num_pages=inp["lat_pool"].shape[0])
        lat = lat_rows(inp["lat_pool"], inp["lat_fmt"], P, rows[rows >= 0])
        o, lse = sparse_mla(C.bf16(inp["q_mla"][t]), lat, inp["sm_scale"])
        out["t"].append(t)
        out["scores"].append(sc if want_scores else None)
        out["idx"].append(sel)
        out["tau"].append(tau)
        out["rows"].append(rows)
        out["o"].append(o)
        out["lse"].append(lse)
    return out


def mla_on_rows(inp: dict, rows: np.ndarray, tokens=None):
    """Sparse MLA alone, on given physical rows per query row ([T,k]); entries
    < 0 or past the pool's last row name no row and are skipped."""
    T = rows.shape[0]
    tokens = range(T) if tokens is None else tokens
    os, lses = [], []
    n_rows = inp["lat_pool"].shape[0] * inp["P"]
    for t in tokens:
        rr = rows[t][(rows[t] >= 0) & (rows[t] < n_rows)]
        lat = lat_rows(inp["lat_pool"], inp["lat_fmt"], inp["P"], rr)
        o, lse = sparse_mla(C.bf16(inp["q_mla"][t]), lat, inp["sm_scale"])
        os.append(o)
        lses.append(lse)
    return np.stack(os), np.stack(lses)
