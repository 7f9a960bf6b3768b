"""Pins of the sharded top-k merge oracle (oracle/merge.py).

Checked against things other than itself: a pure-Python brute force of the
unsharded top-k (sorted over (-score, index) tuples), a pure-Python re-count
of which shards must re-send, two hand-worked rows whose flags and results are
written out below, and the closed forms of the exchange volume.
"""
import random

import numpy as np
import pytest

from oracle import merge as M

pytestmark = pytest.mark.filterwarnings("ignore")


def brute_topk(row, vis, k):
    order = sorted(range(vis), key=lambda s: (-float(row[s]), s))
    return sorted(order[:min(k, vis)])


def brute_flags(row, vis, W, k, cand):
    """First-exchange detection written out with Python sorting only."""
    K = min(k, vis)
    sent = []
    for r in range(W):
        mine = list(range(r, vis, W))
        mine.sort(key=lambda s: (-float(row[s]), s))
        sent.append(mine[:cand])
    union = [s for lst in sent for s in lst]
    union.sort(key=lambda s: (-float(row[s]), s))
    top = set(union[:K])
    flags = []
    for r in range(W):
        n_r = len(range(r, vis, W))
        flags.append(all(s in top for s in sent[r]) and len(sent[r]) < min(k, n_r))
    return flags


def _rows(seed):
    g = np.random.default_rng(seed)
    yield g.standard_normal(300).astype(np.float32)
    yield g.integers(-3, 4, 300).astype(np.float32)                 # heavy ties
    z = np.zeros(300, np.float32)
    z[g.random(300) < 0.5] = -0.0                                   # +0 / -0 only
    yield z
    b = g.standard_normal(300).astype(np.float32)
    b[::3] += 10.0                                                  # one shard (W=3) holds the top
    yield b


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sharded_equals_brute_force_topk(seed):
    rnd = random.Random(seed)
    for row in _rows(seed):
        for _ in range(12):
            W = rnd.choice([1, 2, 3, 4, 7, 8, 16])
            k = rnd.choice([1, 5, 16, 40, 64])
            vis = rnd.choice([0, 1, 3, W, 37, 150, 300])
            cand = rnd.choice([None, 1, 2, max(1, k // W), k])
            idx, flags, sent = M.sharded_topk(row, vis, W, k, cand)
            assert idx.tolist() == brute_topk(row, vis, k), (W, k, vis, cand)
            c = M.default_cand(k, W) if cand is None else cand
            assert flags.tolist() == brute_flags(row, vis, W, k, c), (W, k, vis, cand)
            n = M.shard_counts(vis, W)
            assert sent[0].tolist() == np.minimum(c, n).tolist()
            assert sent[1].tolist() == np.where(flags, np.minimum(k, n), 0).tolist()


def test_all_equal_scores_flag_every_shard():
    # W=4, k=16, cand=3, vis=100, every score equal: shard r sends r, r+4, r+8;
    # the union holds 12 < 16 candidates, so all are selected and every shard
    # (which sent 3 < min(16, 25)) re-sends; the result is 0..15.
    row = np.ones(100, np.float32)
    idx, flags, sent = M.sharded_topk(row, 100, 4, 16, 3)
    assert flags.tolist() == [True] * 4
    assert idx.tolist() == list(range(16))
    assert sent.tolist() == [[3, 3, 3, 3], [16, 16, 16, 16]]


def test_one_shard_holds_the_top():
    # W=4, k=8, cand=3, vis=1000, score 1 on tokens 0 mod 4, else 0.  First exchange:
    # shard 0 sends 0,4,8 (all selected: flagged); the other five places go to
    # the lowest score-0 indices 1,2,3,5,6 (shards 1,2,3 keep a loser each).
    # After shard 0 re-sends 8 candidates the result is 0,4,...,28.
    row = np.where(np.arange(1000) % 4 == 0, 1.0, 0.0).astype(np.float32)
    idx, flags, sent = M.sharded_topk(row, 1000, 4, 8, 3)
    assert flags.tolist() == [True, False, False, False]
    assert idx.tolist() == list(range(0, 32, 4))
    assert sent[1].tolist() == [8, 0, 0, 0]


def test_decreasing_scores_need_no_resend():
    # score = -s: the top-k are 0..k-1, k/W per shard <= the default cand.
    for W in (2, 4, 8, 16):
        row = -np.arange(5000, dtype=np.float32)
        idx, flags, _ = M.sharded_topk(row, 5000, W, 2048)
        assert not flags.any() and idx.tolist() == list(range(2048))


def test_single_shard_is_plain_topk():
    g = np.random.default_rng(5)
    row = g.standard_normal(3000).astype(np.float32)
    idx, flags, sent = M.sharded_topk(row, 3000, 1, 2048)
    assert idx.tolist() == brute_topk(row, 3000, 2048) and not flags.any()
    assert sent[0, 0] == 2048


def test_exchange_volume_closed_forms():
    # default candidates: ceil(1.5 k / W); at k=2048, W=8 that is 384 per shard,
    # 8 * 384 * 8 B = 24 KiB per row against 8 * 2048 * 8 B for the full lists.
    assert M.default_cand(2048, 8) == 384 and M.default_cand(2048, 1) == 2048
    assert M.default_cand(2048, 3) == 1024
    n = M.shard_counts(1 << 20, 8)
    assert n.tolist() == [131072] * 8
    sent = np.array([[384] * 8, [0] * 8])
    assert M.exchange_bytes(sent) == 24576
    assert M.generic_exchange_bytes(n, 2048) == 131072
    assert M.shard_counts(5, 8).tolist() == [1, 1, 1, 1, 1, 0, 0, 0]
    assert M.shard_counts(17, 4).tolist() == [5, 4, 4, 4]


def test_unshard_inverts_the_interleaved_split():
    g = np.random.default_rng(3)
    for W, vis in ((1, 10), (3, 10), (8, 5), (4, 64)):
        row = g.standard_normal(vis).astype(np.float32)
        parts = M.shard_local(row, vis, W)
        ld = max(1, max(len(p) for p in parts))
        local = np.zeros((W, ld), np.float32)
        for r, p in enumerate(parts):
            local[r, :len(p)] = p
            assert np.array_equal(p, row[r::W])
        assert np.array_equal(M.unshard_row(local, vis, W), row)


def test_batch_form_matches_rows():
    g = np.random.default_rng(9)
    W, T, k = 4, 5, 32
    vis = np.array([0, 7, 100, 257, 400])
    ld = 100
    local = g.standard_normal((W, T, ld)).astype(np.float32)
    idx, count, flags, sent = M.sharded_topk_rows(local, vis, W, k)
    for t in range(T):
        row = M.unshard_row(local[:, t], int(vis[t]), W)
        assert idx[t, :count[t]].tolist() == brute_topk(row, int(vis[t]), k)
        assert (idx[t, count[t]:] == -1).all()
