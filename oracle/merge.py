"""Exact top-k merge across context shards, as a plain NumPy reference.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this package; the product path never imports it.

What it follows (Kimi K3.1 Pro day-0 page, "Long context: decode context
parallel" and "Exact top-k merge with 10x less traffic"): under decode context
parallelism shard r of W stores every W-th token (global token s = j*W + r at
local position j), so each shard can rank only its own tokens.  Each shard
sends a short list of its best candidates with their scores; every receiver
selects the global top-k from the union by radix selection; the merge stays
exact because a shard whose sent candidates might not cover its share of the
global top-k is detected and re-sends its full local top-k for that row.

Readings (where the pages leave a step open):
  * ranking is the one of the unsharded top-k: score descending, ties to the
    lower global index, -0 equal to +0; K_t = min(k, vis_t);
  * a candidate carries the fp32 score and the global index (the pages pack a
    BF16 score and an id into 32 bits; fp32 scores need 64 bits to keep the
    merge exact with respect to the fp32 ranking);
  * a shard sends its min(cand, n_r) best local positions (n_r = its visible
    tokens of the row); the default cand = ceil(1.5 k / W);
  * detection: shard r must re-send when every candidate it sent was selected
    and it sent fewer than min(k, n_r) -- then an unsent token of r might still
    rank inside the global top-k; otherwise every unsent token of r ranks
    below a sent one that lost, so it loses too;
  * one re-send round suffices: a shard that sent its full local top-k holds
    no further member of the global top-k, and adding candidates can only
    raise the selection threshold, so no other shard becomes flagged.
"""
from __future__ import annotations

import numpy as np

from . import dsa as O


def default_cand(k: int, W: int) -> int:
    """Candidates each shard sends per row: ceil(1.5 k / W), at most k."""
    return min(k, -(-3 * k // (2 * W)))


def shard_local(row: np.ndarray, vis: int, W: int):
    """Split the visible prefix of one score row into W interleaved shards:
    shard r gets tokens r, r+W, r+2W, ... (n_r = ceil((vis - r) / W) of them)."""
    return [np.asarray(row[r:vis:W]) for r in range(W)]


def shard_send(local: np.ndarray, r: int, W: int, m: int):
    """A shard's message for one row: its min(m, n_r) best local positions
    (the unsharded ranking restricted to the shard), as (score, global index)
    pairs with the local positions ascending."""
    sel, _ = O.topk(local, m)
    return local[sel], sel * W + r


def merge_select(scores: np.ndarray, gidx: np.ndarray, K: int):
    """The K best of a candidate union by (score desc, global index asc);
    returns a boolean mask over the candidates."""
    order = np.lexsort((gidx, -scores.astype(np.float64)))
    mask = np.zeros(len(scores), dtype=bool)
    mask[order[:K]] = True
    return mask


def sharded_topk(row: np.ndarray, vis: int, W: int, k: int, cand: int | None = None):
    """Top-k of one row through the sharded merge.  Returns (idx ascending
    int64 [K_t], flags bool [W] (shards that re-sent), sent int64 [2, W]
    (candidates each shard sent in the first round and in the re-send))."""
    cand = default_cand(k, W) if cand is None else cand
    K = min(k, vis)
    shards = shard_local(row, vis, W)
    n = np.array([len(s) for s in shards], dtype=np.int64)
    msgs = [shard_send(shards[r], r, W, cand) for r in range(W)]
    sent = np.zeros((2, W), dtype=np.int64)
    sent[0] = [len(m[0]) for m in msgs]

    def select(ms):
        sc = np.concatenate([m[0] for m in ms]) if ms else np.zeros(0, np.float32)
        gi = np.concatenate([m[1] for m in ms]) if ms else np.zeros(0, np.int64)
        owner = np.concatenate([np.full(len(m[0]), r) for r, m in enumerate(ms)])
        mask = merge_select(sc, gi, K)
        chosen = np.bincount(owner[mask], minlength=W)
        return gi[mask], chosen

    picked, chosen = select(msgs)
    full = np.minimum(k, n)
    flags = (chosen == sent[0]) & (sent[0] < full)
    if flags.any():
        for r in np.nonzero(flags)[0]:
            msgs[r] = shard_send(shards[r], r, W, k)
            sent[1, r] = len(msgs[r][0])
        picked, chosen = select(msgs)
        again = (chosen == np.array([len(m[0]) for m in msgs])) & (np.array([len(m[0]) for m in msgs]) < full)
        assert not again.any(), "a second re-send round is never needed"
    return np.sort(picked), flags, sent


def sharded_topk_rows(shard_scores: np.ndarray, tok_vis: np.ndarray, W: int, k: int, cand: int | None = None):
    """Batch form on the shard-local layout [W, T, ld] (shard r's local
    position j of row t at [r, t, j]).  Returns (idx int64 [T, k] with -1
    padding, count [T], flags int32 [T, W], sent [T, 2, W])."""
    T = len(tok_vis)
    idx = np.full((T, k), -1, dtype=np.int64)
    count = np.zeros(T, dtype=np.int64)
    flags = np.zeros((T, W), dtype=np.int32)
    sent = np.zeros((T, 2, W), dtype=np.int64)
    for t in range(T):
        vis = int(tok_vis[t])
        row = unshard_row(shard_scores[:, t, :], vis, W)
        sel, fl, se = sharded_topk(row, vis, W, k, cand)
        idx[t, :len(sel)] = sel
        count[t] = len(sel)
        flags[t] = fl
        sent[t] = se
    return idx, count, flags, sent


def unshard_row(local_rows: np.ndarray, vis: int, W: int) -> np.ndarray:
    """Inverse of the interleaved split: local_rows [W, ld] -> the row's
    first vis scores in global order."""
    row = np.zeros(vis, dtype=local_rows.dtype)
    for r in range(W):
        nr = max(0, -(-(vis - r) // W))
        row[r:vis:W] = local_rows[r, :nr]
    return row


def exchange_bytes(sent: np.ndarray) -> int:
    """Bytes the candidate exchange moves: 8 per candidate sent (fp32 score
    key + 32-bit global index), both rounds."""
    return int(8 * np.asarray(sent).sum())


def generic_exchange_bytes(n_local: np.ndarray, k: int) -> int:
    """Bytes of the generic merge, where every shard sends its full local
    top-k as (fp32 score, int32 id) pairs."""
    return int(8 * np.minimum(k, np.asarray(n_local)).sum())


def shard_counts(vis: int, W: int) -> np.ndarray:
    """n_r = ceil((vis - r) / W) for r < W (0 where r >= vis)."""
    return np.array([max(0, -(-(vis - r) // W)) for r in range(W)], dtype=np.int64)

