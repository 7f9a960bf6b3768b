"""Block-sparse attention of the MSA variant, as a plain NumPy reference.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this package; the product path never imports it.

What it follows (MiniMax M3.1 page, "MSA primer"): the KV cache is cut into
blocks of 128 tokens; a light indexer scores every visible key with one index
query per GQA group against a single index-key head shared by the groups; the
scores are max-pooled to one score per block; exact attention then runs over
the top 16 blocks only, the most recent block always among them, so a query
reads at most 2,048 keys whatever the context length; every query head of a
group attends to exactly its group's blocks.

Readings (where the page leaves a step open; the design notes list them):
  * index score of key s for group g: the plain dot product q_idx[g] . k_s of
    the dequantised 128-d index key (no weights, no ReLU); index keys are
    128 E4M3 bytes per token, unscaled (the page's 128 bytes per token);
  * a block's score is the maximum over its visible keys;
  * selection: the most recent block (the one holding position vis - 1) is
    always kept and the other top_blocks - 1 places go to the best-scoring
    other blocks (ties to the lower block index); with at most top_blocks
    blocks every block is kept; selected blocks are listed ascending;
  * K and V: per token, Hkv heads of 128 E4M3 values each for K, then the
    same for V (2 * Hkv * 128 bytes), each tensor with one fp32 scale;
  * attention: query head h belongs to group h // (Hq / Hkv) and uses that
    group's K and V head; logits sm_scale * q_h . k_s over the visible keys of
    the selected blocks; natural-base softmax; o_h = sum p_s v_s, lse in nats;
  * an absent block (block-table entry < 0 or past the pool) has score -inf
    and its tokens are never attended; a row with no attended token gives
    o = 0 and lse = -inf.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import e4m3

BLOCK = 128
DIM = 128


def index_scores(q_idx: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """q_idx [Hkv, 128], keys [n, 128] (dequantised) -> scores [Hkv, n]."""
    return np.asarray(q_idx, np.float64) @ np.asarray(keys, np.float64).T


def block_max(scores: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """scores [.., n] -> [.., ceil(n / block)]: the maximum of every block."""
    n = scores.shape[-1]
    nb = -(-n // block)
    out = np.full(scores.shape[:-1] + (nb,), -np.inf)
    for b in range(nb):
        out[..., b] = scores[..., b * block:min(n, (b + 1) * block)].max(axis=-1)
    return out


def select_blocks(bscores: np.ndarray, top_blocks: int) -> np.ndarray:
    """Block ids kept for one (row, group): the last block plus the best
    top_blocks - 1 others (score desc, lower id on ties), ascending."""
    nb = len(bscores)
    if nb <= top_blocks:
        return np.arange(nb)
    others = np.arange(nb - 1)
    order = np.lexsort((others, -bscores[:-1]))
    keep = np.concatenate([others[order[:top_blocks - 1]], [nb - 1]])
    return np.sort(keep)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """q [G, 128], k / v [m, 128] -> o [G, 128], lse [G]."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], DIM)), np.full(q.shape[0], -math.inf)
    lg = sm_scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    mx = lg.max(axis=1)
    e = np.exp(lg - mx[:, None])
    z = e.sum(axis=1)
    return (e @ np.asarray(v, np.float64)) / z[:, None], mx + np.log(z)


def present(block_table: np.ndarray, r: int, nb: int, pool_blocks: int) -> np.ndarray:
    """Which of request r's first nb logical blocks map into the pool."""
    pages = block_table[r, :nb]
    return (pages >= 0) & (pages < pool_blocks)


def request_index_keys(idx_pool: np.ndarray, block_table: np.ndarray, r: int, n: int) -> np.ndarray:
    """Dequantised index keys of tokens 0..n-1 of request r: [n, 128] (zeros
    for tokens of absent blocks).  The pool is [pool_blocks, 128 * 128] E4M3
    bytes (128 tokens per block)."""
    nb = -(-n // BLOCK)
    ok = present(block_table, r, nb, idx_pool.shape[0])
    pages = np.where(ok, block_table[r, :nb], 0)
    codes = idx_pool[pages].reshape(nb * BLOCK, DIM)
    vals = e4m3(codes)
    vals[np.repeat(~ok, BLOCK)] = 0.0
    return vals[:n]


def request_kv(kv_pool: np.ndarray, block_table: np.ndarray, r: int, blocks: np.ndarray, n: int, hkv: int,
               g: int, k_scale: float, v_scale: float):
    """K and V of group g for the tokens of the given logical blocks that are
    < n, in token order: ([m, 128], [m, 128]).  kv_pool is [pool_blocks,
    128 * 2 * hkv * 128] E4M3 bytes."""
    nb_all = block_table.shape[1]
    ok = present(block_table, r, nb_all, kv_pool.shape[0])
    parts = [np.arange(b * BLOCK, min(n, (b + 1) * BLOCK)) for b in blocks if ok[b]]
    tok = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    per_page = kv_pool.reshape(kv_pool.shape[0], BLOCK, 2, hkv, DIM)
    pages = block_table[r, tok // BLOCK]
    kc = per_page[pages, tok % BLOCK, 0, g]
    vc = per_page[pages, tok % BLOCK, 1, g]
    return k_scale * e4m3(kc), v_scale * e4m3(vc)


def msa_row(inp: dict, t: int):
    """One query row through the whole MSA decode step.  Returns (sel [Hkv,
    top_blocks] with -1 padding, o [Hq, 128], lse [Hq], block scores [Hkv, nb])."""
    r = int(inp["tok_req"][t])
    n = int(inp["tok_vis"][t])
    hkv, hq, top = int(inp["hkv"]), int(inp["hq"]), int(inp["top_blocks"])
    G = hq // hkv
    bt = inp["block_table"]
    keys = request_index_keys(inp["idx_pool"], bt, r, n)
    sc = index_scores(inp["q_idx"][t], keys)
    bs = block_max(sc)
    bs[:, ~present(bt, r, bs.shape[1], inp["idx_pool"].shape[0])] = -np.inf
    sel = np.full((hkv, top), -1, np.int64)
    o = np.zeros((hq, DIM))
    lse = np.zeros(hq)
    for g in range(hkv):
        blocks = select_blocks(bs[g], top)
        sel[g, :len(blocks)] = blocks
        k, v = request_kv(inp["kv_pool"], bt, r, blocks, n, hkv, g, inp["k_scale"], inp["v_scale"])
        og, lg = attention(inp["q"][t, g * G:(g + 1) * G], k, v, inp["sm_scale"])
        o[g * G:(g + 1) * G] = og
        lse[g * G:(g + 1) * G] = lg
    return sel, o, lse, bs
